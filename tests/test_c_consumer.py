"""The C ABI used from plain C: a C99 program compiled with gcc against
include/atw.h and linked to libatw.so calls the host-only entry points and
prints the integer windows, the pruned-term counts and the validation path;
the values must equal the fp64 oracle's bit for bit.  No GPU is touched."""

import os
import shutil
import subprocess

import pytest

import oracle
from rope_frequency_pair_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

C_SRC = r"""
#include <stdio.h>
#include "atw.h"

int main(void) {
  int64_t w[64];
  int64_t pruned = 0, total = 0;
  if (atw_window_widths(64, 1e4, 4.0, 1, w) != ATW_OK) return 1;
  for (int r = 0; r < 32; ++r) printf("%lld ", (long long)w[r]);
  printf("\n");
  if (atw_pruned_terms(1024, 1024, 0, 64, 1e4, 4.0, 1, 1, &pruned, &total) != ATW_OK) return 2;
  printf("%lld %lld\n", (long long)pruned, (long long)total);
  if (atw_pruned_terms(131072, 131072, 0, 128, 5e5, 8.0, 1, 1, &pruned, &total) != ATW_OK) return 3;
  printf("%lld %lld\n", (long long)pruned, (long long)total);
  /* an odd head_dim is rejected before anything runs, with a message */
  int e = atw_window_widths(63, 1e4, 4.0, 1, w);
  printf("%d %s\n", e, atw_last_error()[0] ? "message" : "none");
  printf("%s\n", atw_version());
  return 0;
}
"""


@pytest.fixture(scope="module")
def program(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    lib = binding.LIB_PATH
    if not os.path.exists(lib):
        pytest.skip("libatw.so is not built")
    d = tmp_path_factory.mktemp("c_consumer")
    src = d / "main.c"
    src.write_text(C_SRC)
    exe = d / "main"
    libdir = os.path.dirname(lib)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), str(src),
                    "-o", str(exe), f"-L{libdir}", "-latw", f"-Wl,-rpath,{libdir}"], check=True)
    return str(exe)


def test_c_program_matches_oracle(program):
    out = subprocess.run([program], capture_output=True, text=True, check=True, timeout=120).stdout.split("\n")
    widths = [int(x) for x in out[0].split()]
    assert widths == [int(x) for x in oracle.window_widths(64, 1e4, 4.0)]
    assert tuple(int(x) for x in out[1].split()) == oracle.pruned_terms(1024, 1024, 0, 64, 1e4, 4.0)
    assert tuple(int(x) for x in out[2].split()) == oracle.pruned_terms(131072, 131072, 0, 128, 5e5, 8.0)
    code, msg = out[3].split()
    assert int(code) == binding.ATW_EINVAL and msg == "message"
    assert out[4].startswith("atw ")
