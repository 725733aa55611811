"""Host-side logic of the kernels, checked on the CPU: the workgroup -> tile
remap is a bijection for every grid shape, and the LDS chunk swizzles keep
their bank-spreading properties.  A small host program including the same
device header (gemm_device.hpp) is compiled with hipcc and run here; nothing
touches a GPU.

Also the pages' own worked example of bank arithmetic ("[CUDA 优化实战] hgemm -
超越 cuBLAS", section 4: warp 0 writing a 128-wide half-precision C tile, 32
banks of 4 bytes) is reproduced by the same bank model used for our LDS
patterns (tests/golden/p1_swizzle_c_warp0.txt)."""
import os
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")

HARNESS = r"""
#include "gemm_device.hpp"
#include <cstdio>
#include <vector>
using namespace gemm;
int main() {
  // remap bijection over many grids and strip widths
  for (int tm = 1; tm <= 40; ++tm)
    for (int tn = 1; tn <= 40; ++tn)
      for (int g = 1; g <= 9; ++g) {
        int n = tm * tn;
        std::vector<int> seen(n, 0);
        for (int b = 0; b < n; ++b) {
          int m_, n_;
          tile_coords(b, n, tm, tn, g < tm ? g : tm, m_, n_);
          if (m_ < 0 || m_ >= tm || n_ < 0 || n_ >= tn) { printf("OUT %d %d %d %d\n", tm, tn, g, b); return 1; }
          seen[m_ * tn + n_]++;
        }
        for (int i = 0; i < n; ++i) if (seen[i] != 1) { printf("DUP %d %d %d\n", tm, tn, g); return 1; }
      }
  // big grids used by the benchmark shapes
  int shapes[][2] = {{16, 16}, {17, 16}, {64, 64}, {256, 1}, {33, 32}, {1, 300}};
  for (auto &s : shapes) {
    int n = s[0] * s[1];
    std::vector<int> seen(n, 0);
    for (int b = 0; b < n; ++b) { int m_, n_; tile_coords(b, n, s[0], s[1], s[0] < 4 ? s[0] : 4, m_, n_);
      if (m_ < 0 || m_ >= s[0] || n_ < 0 || n_ >= s[1]) { printf("OUT big\n"); return 1; }
      seen[m_ * s[1] + n_]++; }
    for (int i = 0; i < n; ++i) if (seen[i] != 1) { printf("DUP big\n"); return 1; }
  }
  // 16x16 tiles: each XCD's 32 consecutive workgroups cover a 4 x 8 block of tiles
  for (int x = 0; x < 8; ++x) {
    int mlo = 99, mhi = -1, nlo = 99, nhi = -1;
    for (int p = 0; p < 32; ++p) { int m_, n_; tile_coords(x + 8 * p, 256, 16, 16, 4, m_, n_);
      mlo = m_ < mlo ? m_ : mlo; mhi = m_ > mhi ? m_ : mhi; nlo = n_ < nlo ? n_ : nlo; nhi = n_ > nhi ? n_ : nhi; }
    if (mhi - mlo != 3 || nhi - nlo != 7) { printf("XCD block %d: rows %d-%d cols %d-%d\n", x, mlo, mhi, nlo, nhi); return 1; }
  }
  // swizzles: 8 consecutive rows, and 8 rows 8 apart, hit 8 distinct chunks
  for (int base = 0; base < 512; base += 8)
    for (int c = 0; c < 8; ++c) {
      int m1 = 0, m2 = 0;
      for (int r = 0; r < 8; ++r) { m1 |= 1 << (c ^ swz8(base + r)); m2 |= 1 << (c ^ swz8((base / 8) * 64 % 512 + 8 * r + (base % 8))); }
      if (m1 != 255 || m2 != 255) { printf("swz8 %d %d\n", base, c); return 1; }
    }
  for (int base = 0; base < 512; base += 8)
    for (int c = 0; c < 4; ++c) {
      // two 64-byte rows per 128 bytes: rows base..base+7 at chunk c cover 8 distinct 16-byte slots
      int m = 0;
      for (int r = 0; r < 8; ++r) m |= 1 << (((base + r) & 1) * 4 + (c ^ swz4(base + r)));
      if (m != 255) { printf("swz4 %d %d\n", base, c); return 1; }
    }
  // strided K walks (the few-row kernel): 16 waves, 7 groups each per round, up
  // to 8 rows per group; for K up to the library's limit 2^31 - 2^16 every
  // index formed stays below 2^31 and indexes past the last group read as K
  {
    const long long lim = (1LL << 31) - (1LL << 16);
    const int Ks[] = {1, 7, 8, 9, 1000, 4100, (int)lim - 1, (int)lim};
    for (int K : Ks)
      for (int per : {4, 8}) {
        const int ngroups = (int)(((long long)K + per - 1) / per);
        const int first = ngroups > 200 ? ngroups - 200 : 0;
        for (int g0 = first; g0 < ngroups; ++g0)
          for (int u = 0; u < 7; ++u)
            for (int r = 0; r < per; ++r) {
              const long long g = (long long)g0 + 16LL * u;
              const int k = group_elem(g0 + 16 * u, ngroups, per, r, K);
              const long long want = g < ngroups ? g * per + r : K;
              if (k != want || k < 0) { printf("group_elem K=%d g=%lld r=%d: %d\n", K, g, r, k); return 1; }
            }
      }
  }
  printf("OK\n");
  return 0;
}
"""


def test_remap_and_swizzles_host_harness():
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "h.hip"), os.path.join(d, "h")
        open(src, "w").write(HARNESS)
        r = subprocess.run(["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O1", "-std=c++17",
                            "-I", os.path.join(ROOT, "dense_gemm_13_amd", "csrc"), src, "-o", exe],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        out = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0 and out.stdout.strip() == "OK", out.stdout + out.stderr


def bank_of(byte_addr: int, banks: int = 32, width: int = 4) -> int:
    return (byte_addr // width) % banks


def _golden(name):
    kv = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if line and not line.startswith("#") and ":" in line:
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    return kv


def test_pages_swizzle_c_worked_example():
    g = _golden("p1_swizzle_c_warp0.txt")
    rows = [int(x) for x in g["rows"].split(",")]
    cols = [int(x) for x in g["cols"].split(",")]
    width = int(g["tile_width_elems"])
    esize = int(g["elem_bytes"])
    # the text's bank formula: (row*128 + col)*2/4 % 32 == (col/2) % 32
    naive = [bank_of((r * width + c) * esize) for r, c in zip(rows, cols)]
    assert all(b == (c // 2) % 32 for b, c in zip(naive, cols))
    # without the swizzle every row lands on the same 4 banks: 8-way conflict
    assert max(naive.count(b) for b in set(naive)) == int(g["naive_conflict_ways"])
    # with col ^ ((row & 7) << 3) the 32 lanes hit 32 distinct banks
    swz = [bank_of((r * width + (c ^ ((r & 7) << 3))) * esize) for r, c in zip(rows, cols)]
    assert len(set(swz)) == int(g["swizzled_distinct_banks"])


def test_pages_benchmark_table_metric():
    """TFLOP/s = 2MNK / time reproduces every row of the pages' 4096^3 table."""
    import bench
    kv = _golden("p1_hgemm_4096_table.txt")
    torch_ms = float(kv["torch"].split(",")[0])
    for name, val in kv.items():
        if name.startswith(("M", "N", "K")) or name == "source":
            continue
        ms, tf, speedup = (float(x) for x in val.split(","))
        assert abs(bench.tflops(4096, 4096, 4096, ms * 1e-3) - tf) < 0.006, name
        assert abs(torch_ms / ms - speedup) < 0.006, name


def test_pages_flop_arithmetic():
    """4096^3 x 2 ~ 137.4 GFLOP, 4.6 ms at 30 TFLOP/s (the pages' section 1.2 example)."""
    import bench
    kv = _golden("p3_flop_example.txt")
    flops = 2 * 4096 ** 3
    assert abs(flops / 1e9 - float(kv["gflop"])) < 0.05
    assert abs(flops / (float(kv["tflops"]) * 1e12) * 1e3 - float(kv["ms"])) < 0.05
    assert abs(bench.tflops(4096, 4096, 4096, float(kv["ms"]) * 1e-3) - float(kv["tflops"])) < 0.2


def test_pages_tiled_intensity():
    """Block tiling of C moves MN + MNK(BM+BN)/(BM*BN) elements; for large K the
    intensity 2MNK / that tends to 2/(1/BM + 1/BN), which is b for BM = BN = b."""
    kv = _golden("p2_tiled_intensity.txt")
    for b in (int(x) for x in kv["b"].split(",")):
        M = N = K = 1 << 16
        traffic = M * N + M * N * K * (2 * b) / (b * b)
        intensity = 2 * M * N * K / traffic
        assert abs(intensity - b) / b < 0.01
