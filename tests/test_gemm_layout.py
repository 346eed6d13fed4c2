"""Host checks of LDS layouts used by the kernels: compiles a checker against
the kernel's index header with the host C++ compiler and runs it (every LDS
placement, every operand fetch, bank conflicts, and the offset arithmetic the
kernel derives from them)."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_gemm_tile_layouts(tmp_path):
    exe = tmp_path / "gemm_layout_check"
    subprocess.run(["g++", "-O1", "-std=c++17", "-I", os.path.join(ROOT, "adjoint_gradients_amd", "csrc"),
                    "-o", str(exe), os.path.join(ROOT, "tests", "gemm_layout_check.cpp")], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "layout OK" in out.stdout


def test_reduction_buffer_layout(tmp_path):
    """Placement of the reverse walk's channel-sum transpose buffer
    (csrc/red_layout.hpp): bijective, each lane reads its own row segment, and
    the unpadded layout is free of LDS bank conflicts."""
    exe = tmp_path / "red_layout_check"
    subprocess.run(["g++", "-O1", "-std=c++17", "-I", os.path.join(ROOT, "adjoint_gradients_amd", "csrc"),
                    "-o", str(exe), os.path.join(ROOT, "tests", "red_layout_check.cpp")], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "layout OK" in out.stdout
