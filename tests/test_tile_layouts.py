"""Host checks of the tile-ordered E8M0 scale layouts the attention kernel reads
(``key_tile_byte`` / ``dim_tile_byte`` in csrc/fsa_internal.h), compiled for the
host with g++ (no GPU).

* Each layout is a bijection: every (key row, D block) of a 128-key tile, or
  (output row, key block), owns exactly one byte of the tile.
* The key order it encodes matches the 32x32x64 product's output layout (lane
  (h, n), register i holds row 8(i/4) + 4h + i%4): in block b of a 64-key chunk,
  register i of lane half h is key 32h + 16b + i (FP6/FP4) or 32b + 16h + i (FP8),
  which is what lets a lane feed its 32 outputs to the P V product in place.
* The byte of (key, D block 2c + h) sits in the D/16 bytes (8 at D=128, 4 at D=64) of
  lane 32h + rho at position u*2nd + b*nd + c, and the byte of (row d, key
  block 2u + h) in those of lane 32h + d%32 at u*D/32 + d/32.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "softmax_mx_quantize_amd", "csrc")

PROGRAM = r"""
#include "fsa_internal.h"
#include <cstdio>
#include <vector>
using fsa::key_tile_byte; using fsa::dim_tile_byte;
static int fails = 0;
#define CHECK(c, ...) do { if (!(c)) { if (fails++ < 10) std::printf(__VA_ARGS__); } } while (0)
int main() {
  for (int d : {64, 128}) {
    const int nd = d / 64, nbk = d / 16, nbv = d / 16;
    for (int bits : {8, 6, 4}) {
      std::vector<int> seen(128 * d / 32, 0);
      for (int rl = 0; rl < 128; ++rl)
        for (int blk = 0; blk < d / 32; ++blk) {
          const int by = key_tile_byte(rl, blk, d, bits);
          CHECK(by >= 0 && by < 128 * d / 32, "K range d=%d bits=%d rl=%d blk=%d -> %d\n", d, bits, rl, blk, by);
          if (by >= 0 && by < 128 * d / 32) seen[by]++;
        }
      for (size_t i = 0; i < seen.size(); ++i) CHECK(seen[i] == 1, "K byte %zu hit %d times (d=%d bits=%d)\n", i, seen[i], d, bits);
      // output register i of lane (h, n) in block b of chunk u holds A row
      // 8(i/4) + 4h + i%4; its key must be the one the kernel assumes
      for (int u = 0; u < 2; ++u) for (int b = 0; b < 2; ++b) for (int h = 0; h < 2; ++h)
        for (int i = 0; i < 16; ++i) {
          const int rho = 8 * (i / 4) + 4 * h + i % 4;
          const int key = 64 * u + (bits == 8 ? 32 * b + 16 * h + i : 32 * h + 16 * b + i);
          for (int c = 0; c < nd; ++c)
            for (int hs = 0; hs < 2; ++hs) {
              const int want = (32 * hs + rho) * nbk + u * 2 * nd + b * nd + c;
              const int got = key_tile_byte(key, 2 * c + hs, d, bits);
              CHECK(got == want, "K order d=%d bits=%d u=%d b=%d h=%d i=%d c=%d hs=%d: %d != %d\n",
                    d, bits, u, b, h, i, c, hs, got, want);
            }
        }
    }
    std::vector<int> seen(4 * d, 0);
    for (int dd = 0; dd < d; ++dd)
      for (int kb = 0; kb < 4; ++kb) {
        const int by = dim_tile_byte(dd, kb, d);
        CHECK(by >= 0 && by < 4 * d, "V range d=%d dd=%d kb=%d -> %d\n", d, dd, kb, by);
        if (by >= 0 && by < 4 * d) seen[by]++;
        const int want = (32 * (kb & 1) + dd % 32) * nbv + (kb >> 1) * (d / 32) + dd / 32;
        CHECK(by == want, "V order d=%d dd=%d kb=%d: %d != %d\n", d, dd, kb, by, want);
      }
    for (size_t i = 0; i < seen.size(); ++i) CHECK(seen[i] == 1, "V byte %zu hit %d times (d=%d)\n", i, seen[i], d);
  }
  std::printf("fails %d\n", fails);
  return fails != 0;
}
"""


def test_tile_scale_layouts_are_bijections_in_the_product_order(tmp_path):
    gxx = shutil.which("g++")
    inc = "/opt/rocm/include"
    if gxx is None or not os.path.isdir(inc):
        pytest.skip("g++ or the ROCm headers are not available")
    src = tmp_path / "layouts.cpp"
    src.write_text(PROGRAM)
    exe = tmp_path / "layouts"
    subprocess.run([gxx, "-std=c++17", "-O1", "-D__HIP_PLATFORM_AMD__", "-I", inc, "-I", CSRC,
                    str(src), "-o", str(exe)], check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout
    assert "fails 0" in r.stdout
