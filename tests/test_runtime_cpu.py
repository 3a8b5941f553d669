"""The binding and PyTorch share one HIP runtime, whatever the import order.

PyTorch ships its own libamdhip64; the library links libamdhip64.so.7.  If
two copies were mapped into one process, torch's streams would be foreign to
the library's launches.  Loading the library through the binding before torch
is imported must still leave exactly one copy mapped (checked on the CPU: the
runtime loads without a GPU)."""

import subprocess
import sys
import textwrap

import pytest

import exact_attention_121_amd as ea


def _mapped_hip_runtimes(code: str) -> list[str]:
    prog = textwrap.dedent(code) + textwrap.dedent('''
        paths = set()
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    paths.add(line.split()[-1])
        print("\\n".join(sorted(paths)))
    ''')
    out = subprocess.run([sys.executable, "-c", prog], capture_output=True, text=True, timeout=300,
                         cwd=str(__import__("pathlib").Path(__file__).resolve().parents[1]))
    assert out.returncode == 0, out.stderr[-2000:]
    return [line for line in out.stdout.splitlines() if line.strip()]


@pytest.mark.parametrize("order", ["library_first", "torch_first"])
def test_one_hip_runtime_in_the_process(order):
    try:
        ea.load_library()
    except RuntimeError as e:  # not built
        pytest.skip(str(e))
    if order == "library_first":
        code = """
            import exact_attention_121_amd as ea
            ea.load_library()
            import torch
        """
    else:
        code = """
            import torch
            import exact_attention_121_amd as ea
            ea.load_library()
        """
    paths = _mapped_hip_runtimes(code)
    assert len(paths) == 1, f"{order}: HIP runtimes mapped: {paths}"
