"""The C ABI (CPU only): the library loads, exports every declared entry point,
and the binding's ctypes structures have the header's layout."""
import ctypes
import os
import re
import subprocess

import pytest

from spgemm_irregular_matrices_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spgemm.h")


def _declared():
    src = open(HEADER).read()
    return re.findall(r"SPGEMM_API\s+[\w\s\*]+?\b(spgemm_\w+)\s*\(", src)


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert set(names) == set(binding.EXPORTS)
    lib = binding.load()
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for code in range(-11, 1):
        s = binding.status_string(code)
        assert s and s != "unknown status"
    assert binding.status_string(-99) == "unknown status"


def test_struct_layout_matches_header(tmp_path):
    prog = tmp_path / "layout.c"
    prog.write_text(r'''
#include <stddef.h>
#include <stdio.h>
#include "spgemm.h"
int main(void) {
  printf("%zu %zu %zu %zu\n", sizeof(spgemm_csr), sizeof(spgemm_options),
         sizeof(spgemm_stats), sizeof(spgemm_debug_matrix));
  printf("%zu %zu %zu %zu %zu\n", offsetof(spgemm_stats, phase_ms), offsetof(spgemm_stats, lds_bytes),
         offsetof(spgemm_options, max_batch_products), offsetof(spgemm_options, symbolic_mode),
         offsetof(spgemm_options, numeric_mode));
  printf("%zu %zu %zu %zu\n", offsetof(spgemm_stats, numeric_path), offsetof(spgemm_stats, f_u_le),
         offsetof(spgemm_stats, gamma), offsetof(spgemm_options, workspace_limit_bytes));
  return 0;
}''')
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-I", os.path.join(ROOT, "include"), str(prog), "-o", str(exe)])
    out = subprocess.check_output([str(exe)]).decode().split()
    sizes = [int(x) for x in out]
    assert sizes[0] == ctypes.sizeof(binding.CSRStruct)
    assert sizes[1] == ctypes.sizeof(binding.Options)
    assert sizes[2] == ctypes.sizeof(binding.Stats)
    assert sizes[3] == ctypes.sizeof(binding.DebugMatrix)
    assert sizes[4] == binding.Stats.phase_ms.offset
    assert sizes[5] == binding.Stats.lds_bytes.offset
    assert sizes[6] == binding.Options.max_batch_products.offset
    assert sizes[7] == binding.Options.symbolic_mode.offset
    assert sizes[8] == binding.Options.numeric_mode.offset
    assert sizes[9] == binding.Stats.numeric_path.offset
    assert sizes[10] == binding.Stats.f_u_le.offset
    assert sizes[11] == binding.Stats.gamma.offset
    assert sizes[12] == binding.Options.workspace_limit_bytes.offset


def test_no_gpu_call_fails_loudly():
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("GPU present")
    with pytest.raises(Exception):
        binding.Plan()
