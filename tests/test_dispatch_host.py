"""The dense GEMM's shape -> kernel predicate (csrc/nvfp4_dispatch.h), compiled
with the host C++ compiler and checked on the CPU: which kernel each shape
and alignment reaches, and that no path is chosen whose 32-bit buffer
offsets would wrap (the rows one launch reads, weights and activations
both, must stay below 4 GiB)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "nvfp4_block_scaled_gemm_amd", "csrc")

DRIVER = r"""
#include <stdio.h>
#include <stdlib.h>
#include "nvfp4_dispatch.h"
int main(int argc, char** argv) {
  // argv: M N K q16 s8 s16 (same alignment for both operands)
  long long M = atoll(argv[1]), N = atoll(argv[2]), K = atoll(argv[3]);
  nvfp4::OperandAlign al{argv[4][0] == '1', argv[5][0] == '1', argv[6][0] == '1'};
  const bool nvfp4_out = argc > 7 && argv[7][0] == '1';
  printf("%d\n", (int)nvfp4::gemm_path(M, N, K, al, al, nvfp4_out));
  return 0;
}
"""

LDS, DECODE, MFMA, GENERIC, ROWS = 0, 1, 2, 3, 4


@pytest.fixture(scope="module")
def path_of(tmp_path_factory):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    d = tmp_path_factory.mktemp("dispatch")
    src, exe = d / "driver.cpp", d / "driver"
    src.write_text(DRIVER)
    subprocess.run([cxx, "-std=c++17", "-O1", "-I", CSRC, str(src), "-o", str(exe)], check=True)

    def run(M, N, K, q16=True, s8=True, s16=True, nvfp4_out=False):
        out = subprocess.run([str(exe), str(M), str(N), str(K), str(int(q16)), str(int(s8)),
                              str(int(s16)), str(int(nvfp4_out))], check=True,
                             capture_output=True, text=True)
        return int(out.stdout)
    return run


@pytest.mark.parametrize("M,N,K,expect", [
    (1, 8192, 8192, ROWS), (4, 8192, 8192, ROWS), (5, 8192, 8192, LDS), (16, 8192, 8192, LDS),
    (32, 8192, 8192, LDS), (4, 8192, 4096, LDS), (4, 3, 8192, ROWS),
    (1, 8192, 2048, LDS), (3, 1000, 16384, LDS),
    (33, 8192, 8192, DECODE), (64, 8192, 8192, DECODE), (96, 8192, 8192, DECODE),
    (97, 8192, 8192, MFMA), (128, 8192, 8192, MFMA), (100, 40, 256, DECODE),
    (4096, 8192, 8192, MFMA), (16, 512, 512, DECODE), (16, 200, 1536, DECODE),
    (5, 7, 16, GENERIC), (33, 96, 48, GENERIC), (3, 100, 0, GENERIC),
    (1, 1, 1024, LDS), (32, 1, 2048, LDS),
])
def test_shape_to_kernel(path_of, M, N, K, expect):
    assert path_of(M, N, K) == expect


def test_nvfp4_output_avoids_the_whole_row_kernel(path_of):
    """Its chunks hold 4 output columns, not whole 16-column blocks."""
    assert path_of(4, 8192, 8192, nvfp4_out=True) == LDS
    assert path_of(1, 8192, 8192, nvfp4_out=True) == LDS


def test_alignment_steers_away_from_the_fast_paths(path_of):
    assert path_of(16, 8192, 8192, s16=False) == DECODE      # 16-byte scale DMAs need s16
    assert path_of(16, 8192, 8192, s8=False, s16=False) == GENERIC
    assert path_of(4096, 8192, 8192, q16=False) == GENERIC


def test_activation_rows_bound_the_32_bit_offsets(path_of):
    """Few weight rows but K so large that 64 activation rows pass 4 GiB:
    the decode paths (which address a pass's activation rows with 32-bit
    offsets) must not be chosen."""
    K = 1 << 27                      # 64 MiB of nibbles per row
    assert path_of(64, 2, K) == GENERIC        # 64 rows = 4 GiB of activations
    assert path_of(32, 2, K) == LDS            # 2 GiB: fits
    assert path_of(4, 1 << 20, 8192) == GENERIC    # weights of exactly 4 GiB
    assert path_of(4, (1 << 20) - 1, 8192) == ROWS  # 4 KB less: fits
    assert path_of(63, 2, K) == GENERIC
    assert path_of(33, 2, 1 << 26) == DECODE   # 33 rows x 32 MiB: fits
