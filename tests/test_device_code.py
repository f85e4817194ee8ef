"""Device code of libtp_linear.so: no kernel may use per-lane scratch memory.

Every HIP source is compiled for gfx950 to device assembly (no GPU needed), and
the code-object metadata of every kernel instance is read: a non-zero
``.private_segment_fixed_size`` means the compiler spilled registers to scratch
memory, which costs memory traffic in the inner loops and is not allowed for
any instance the library can launch.
"""
import glob
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tensor_sharded_linear_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def kernel_resources(src, tmp_path):
    """[(kernel symbol, private segment bytes, vgpr count)] for every kernel in src."""
    from tensor_sharded_linear_amd.build import FLAGS
    flags = [f for f in FLAGS if f not in ("-shared", "-fPIC")]
    out = tmp_path / (os.path.basename(src) + ".s")
    cmd = [HIPCC, *flags, "--cuda-device-only", "-S", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           src, "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    text = out.read_text()
    # the AMDGPU metadata block lists .name, .private_segment_fixed_size, .vgpr_count per kernel
    kernels = []
    for block in re.split(r"\n\s+- \.", text.split("amdhsa.kernels:")[1]):
        name = re.search(r"\.name:\s+(\S+)", block)
        priv = re.search(r"\.private_segment_fixed_size:\s+(\d+)", block)
        vgpr = re.search(r"\.vgpr_count:\s+(\d+)", block)
        if name and priv:
            kernels.append((name.group(1), int(priv.group(1)), int(vgpr.group(1)) if vgpr else -1))
    return kernels


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc is not installed")
@pytest.mark.parametrize("src", SOURCES, ids=[os.path.basename(s) for s in SOURCES])
def test_no_kernel_spills_to_scratch(src, tmp_path):
    kernels = kernel_resources(src, tmp_path)
    text = open(src).read()
    if "__global__" in text:
        assert kernels, f"no kernel metadata found for {src}"
    spilled = [(n, p) for n, p, _ in kernels if p != 0]
    assert not spilled, f"kernels with scratch (private segment) memory: {spilled}"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc is not installed")
def test_every_gemm_instance_is_compiled_and_checked(tmp_path):
    """The tiled GEMM has 2 output types x bias or not, times 5 tile heights x 2 tile widths
    for each of the 2 plain epilogues (none, GELU) and 3 heights x 1 width for SwiGLU: 92
    instances.  The 192- to 256-row tiles (48 instances of the plain epilogues, 12 of SwiGLU)
    are the four-wave kernel, the 64- and 128-row tiles (32) the eight-wave one."""
    kernels = kernel_resources(os.path.join(CSRC, "gemm_bf16.hip"), tmp_path)
    eight = [n for n, _, _ in kernels if "gemm_bf16_nt_kernel" in n]
    four = [n for n, _, _ in kernels if "gemm4_bf16_nt_kernel" in n]
    assert len(eight) == 32 and len(four) == 60, (eight, four)


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc is not installed")
def test_every_split_k_instance_is_compiled_and_checked(tmp_path):
    """The split-K kernel for up to 128 rows has 6 row-block counts (1-4, 6, 8) x 2 output
    types x bias or not, times 1-3 weight blocks for each of the 2 plain epilogues (none,
    GELU) and 2 (gate, up) for SwiGLU: 168 instances, none spilling."""
    kernels = kernel_resources(os.path.join(CSRC, "gemm_narrow.hip"), tmp_path)
    narrow = [(n, p) for n, p, _ in kernels if "gemm_narrow_kernel" in n]
    assert len(narrow) == 168, [n for n, _ in narrow]
    assert all(p == 0 for _, p in narrow)


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc is not installed")
def test_four_wave_gemm_moves_no_accumulator_among_its_mfmas(tmp_path):
    """The four-wave GEMM writes its MFMAs as inline assembly, so the compiler's hazard checks
    do not see them: an accumulator read, written or moved by a compiler-made instruction
    between the first MFMA and the wait that follows the last one could see a result the MFMA
    has not written yet.  The kernel's single uniform loop body leaves the compiler no reason
    for such a move; this checks every instance's device assembly for one."""
    from tensor_sharded_linear_amd.build import FLAGS
    flags = [f for f in FLAGS if f not in ("-shared", "-fPIC")]
    out = tmp_path / "gemm_bf16.s"
    cmd = [HIPCC, *flags, "--cuda-device-only", "-S", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "gemm_bf16.hip"), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    text = out.read_text()
    checked, bad = 0, []
    for m in re.finditer(r"^(\S*gemm4_bf16_nt_kernel\S*):", text, re.M):
        body = text[m.end():text.index("s_endpgm", m.end())].splitlines()
        first = next(i for i, line in enumerate(body) if "v_mfma" in line)
        wait = next(i for i, line in enumerate(body) if "s_nop 7" in line and i > first)
        moves = [line.strip() for line in body[first:wait] if re.search(r"v_accvgpr_(read|write|mov)", line)]
        checked += 1
        if moves:
            bad.append((m.group(1), len(moves), moves[:2]))
    assert checked == 60, checked
    assert not bad, bad
