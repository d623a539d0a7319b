"""Properties of the compiled decode kernels that the tests on the GPU do not
show: compiles the library's HIP sources to gfx950 assembly (no GPU needed)
and reads each decode kernel's resource descriptor and code.

  * no scratch: a register spill would put scratch traffic into the row loop;
  * at most 168 VGPRs, the count at which three waves fit per SIMD: the plan
    assumes three resident waves per SIMD, and a 12-wave workgroup cannot
    launch with fewer;
  * MFMA in every decode kernel, and no packed-fp32 instruction anywhere (the
    build turns them off).
"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not installed")
    from decode_attention_offloaded_amd import build as kb
    d = tmp_path_factory.mktemp("isa")
    text = []
    for src in kb.HIP_SOURCES:  # every HIP source of the library, with the library's flags
        out = d / (src + ".s")
        cmd = ([HIPCC] + kb.COMMON + ["--offload-arch=" + kb.ARCH] + kb.CODE_OBJECT + kb.NO_PACKED_FP32 +
               kb.KERNARG_PRELOAD + kb.MFMA_VGPR + ["--cuda-device-only", "-S", "-o", str(out),
                                                   os.path.join(kb.CSRC, src)])
        subprocess.run(cmd, check=True, capture_output=True)
        text.append(out.read_text())
    return "\n".join(text)


def _kernels(text):
    """name -> (descriptor text, code text) for every decode kernel."""
    out = {}
    for m in re.finditer(r"\.amdhsa_kernel (\S+)\n(.*?)\.end_amdhsa_kernel", text, re.S):
        name = m.group(1)
        if "decode_kernel" not in name:
            continue
        code = re.search(r"\n%s:[^\n]*\n(.*?)\n\.Lfunc_end" % re.escape(name), text, re.S)
        out[name] = (m.group(2), code.group(1) if code else "")
    return out


def _field(desc, key):
    return int(re.search(r"\.%s (\d+)" % key, desc).group(1))


def test_every_variant_is_built(asm):
    # head_dim 64/128 x group 1..8 x q8_0/q4_0 V x the load modes each wave
    # count is launched with: 4 waves dword / 16-byte via registers / 16-byte
    # into LDS, 8 waves dword / into LDS, 12 waves dword / via registers
    names = _kernels(asm)
    assert len(names) == 2 * 8 * 2 * (3 + 2 + 2)
    modes = {(int(w), int(m)) for m, w in (re.search(r"decode_kernelILi\d+ELi\dELi\dELi(\d)ELi(\d+)E", n).groups()
                                           for n in names)}
    assert modes == {(4, 0), (4, 1), (4, 2), (8, 0), (8, 2), (12, 0), (12, 1)}


def test_no_scratch_and_waves_per_simd(asm):
    """No spills; 4- and 12-wave kernels fit three waves per SIMD (up to three
    4-wave workgroups, or one 12-wave one, per CU), 8-wave kernels two."""
    for name, (desc, _) in _kernels(asm).items():
        assert _field(desc, "amdhsa_private_segment_fixed_size") == 0, name
        w = int(re.search(r"decode_kernelILi\d+ELi\dELi\dELi\dELi(\d+)E", name).group(1))
        assert _field(desc, "amdhsa_next_free_vgpr") <= (256 if w == 8 else 168), name


def test_mfma_in_every_decode_kernel_and_no_packed_fp32(asm):
    for name, (_, code) in _kernels(asm).items():
        assert "v_mfma_f32_16x16x32_f16" in code and "v_mfma_f32_16x16x16_bf16" in code, name
    assert not re.search(r"v_pk_(add|mul|fma)_f32", asm)
