"""LDS bank check of the large-tile kernels' layouts, on the CPU.

A host program includes dense_gemm_13_amd/csrc/gemm_lds_layout.hpp, the header
whose functions the kernels use for every LDS address, and enumerates the 64
lane addresses of each LDS instruction of the bf16/fp16 (256x256, 128x128 and
128x256 tiles), fp8 (256x256 and 128x128) and fp32 (128x128) kernels: the
fragment reads of the main loops (ds_read_b128, the transposing
ds_read_b64_tr_b16 / ds_read_b64_tr_b8, single-float reads), the staged
epilogues' writes and reads, and the LDS-direct loads.

Two properties are checked:
  * placement: the element each LDS-direct load puts in a slot is the one the
    fragment reads look for there (the swizzles of the writer and of the reader
    agree, every slot is written once);
  * banks: the conflict cycles of every instruction under the LDS model that
    matches gfx950's counters -- reads served 256 bytes per clock (64 banks of
    4 bytes: 16 lanes of a 16-byte read, 32 of an 8-byte read, 64 of a 4-byte
    read per cycle), writes 128 bytes per clock (16 lanes of an 8-byte write
    over 32 banks).  The main loops and epilogues must be conflict-free.

Calibration of the model against SQ_LDS_BANK_CONFLICT on MI355X (bf16 4096^3,
256x256 kernel): 262144 conflict cycles per launch (256 per wave) both with and
without the main loop's 3.1 M LDS reads, i.e. all outside the loop; the model
gives 0 for the loop and exactly 256 per wave for the epilogue's staging writes
as they were laid out before (8-byte half flipped on row bit 4, so in 256-byte
rows chunks c and c + 8 met on the same banks), which the check reproduces
below.  The bank arithmetic itself is the one of "[CUDA 优化实战] hgemm - 超越
cuBLAS" section 4 (bank = 4-byte word index modulo the bank count).
"""
import os
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "dense_gemm_13_amd", "csrc")

HARNESS = r"""
#include "gemm_lds_layout.hpp"
#include <cstdio>
#include <map>
#include <set>
#include <vector>
using namespace gemm;

// Extra cycles of one instruction: lanes served `per_pass` at a time, `width`
// bytes each, `banks` banks of 4 bytes; a pass takes as many cycles as the most
// distinct words any bank holds.
static int extra_cycles(const std::vector<long> &addr, int width, int per_pass, int banks)
{
    int extra = 0;
    for (int p0 = 0; p0 < 64; p0 += per_pass) {
        std::map<int, std::set<long>> words;
        for (int l = p0; l < p0 + per_pass; ++l)
            for (int w = 0; w < width / 4; ++w) {
                const long word = addr[l] / 4 + w;
                words[(int)(word % banks)].insert(word);
            }
        int worst = 0;
        for (auto &kv : words) worst = (int)kv.second.size() > worst ? (int)kv.second.size() : worst;
        extra += worst - 1;
    }
    return extra;
}
static int rd(const std::vector<long> &a, int width) { return extra_cycles(a, width, 256 / width, 64); }
static int wr8(const std::vector<long> &a) { return extra_cycles(a, 8, 16, 32); }

static int failures = 0;
static void report(const char *kernel, const char *what, long instrs, long extra)
{
    printf("BANKS %s | %s | instructions %ld | extra cycles %ld\n", kernel, what, instrs, extra);
}
static void placement(const char *kernel, const char *what, bool ok)
{
    printf("PLACE %s | %s | %s\n", kernel, what, ok ? "ok" : "MISMATCH");
    if (!ok) ++failures;
}

// ------------------------------------------------------------ bf16 / fp16
template <int TBM, int TBN>
static void h16(const char *name)
{
    constexpr int BK = 32, WTM = TBM / 2, WTN = TBN / 2, FFM = WTM / 32, FFN = WTN / 32;
    long ar = 0, ai = 0, br = 0, bi = 0;
    for (int wave = 0; wave < 4; ++wave) {
        const int wm0 = (wave / 2) * WTM, wn0 = (wave % 2) * WTN;
        for (int s = 0; s < BK / 16; ++s) {
            for (int i = 0; i < FFM; ++i) {              // A fragments: ds_read_b128
                std::vector<long> a(64);
                for (int l = 0; l < 64; ++l)
                    a[l] = 2L * lds::h16_a_frag<BK>(wm0 + 32 * i + (l & 31), 2 * s + (l >> 5));
                ar += rd(a, 16); ++ai;
            }
            for (int j = 0; j < FFN; ++j)                 // B fragments: two tr_b16 reads
                for (int hi = 0; hi < 2; ++hi) {
                    std::vector<long> a(64);
                    for (int l = 0; l < 64; ++l) {
                        const int g = l >> 4, w16 = l & 15, r4 = w16 >> 2, c4 = w16 & 3;
                        const int n = wn0 + 32 * j + 16 * (g & 1) + 4 * c4;
                        const int krow = 16 * s + 8 * (g >> 1) + r4 + 4 * hi;
                        if (lds::h16_b_col(r4, n) != lds::h16_b_col(krow, n)) ++failures;
                        a[l] = 2L * (krow * TBN + lds::h16_b_col(r4, n));
                    }
                    br += rd(a, 8); ++bi;
                }
        }
    }
    report(name, "main loop A ds_read_b128 (per K step of 32)", ai, ar);
    report(name, "main loop B ds_read_b64_tr_b16 (per K step of 32)", bi, br);
    // LDS-direct loads: lane t of block b writes base + 1024 b + 16 t; the
    // fragment reads must find (row, logical chunk) exactly there.
    bool ok = true;
    std::set<long> seen;
    for (int b = 0; b < TBM * BK * 2 / 1024; ++b)
        for (int l = 0; l < 64; ++l) {
            int row, chunk;
            lds::h16_a_dma<BK>(b, l, row, chunk);
            const long slot = 1024L * b + 16 * l;
            ok &= slot == 2L * lds::h16_a_frag<BK>(row, chunk) && row < TBM && seen.insert(slot).second;
        }
    placement(name, "A stage: LDS-direct slots = fragment-read addresses", ok && (long)seen.size() == TBM * BK * 2 / 16);
    ok = true; seen.clear();
    for (int b = 0; b < BK * TBN * 2 / 1024; ++b)
        for (int l = 0; l < 64; ++l) {
            int row, chunk;
            lds::h16_b_dma<TBN>(b, l, row, chunk);
            const long slot = 1024L * b + 16 * l;
            ok &= slot == 2L * (row * TBN + lds::h16_b_col(row, 8 * chunk)) && row < BK && seen.insert(slot).second;
        }
    placement(name, "B stage: LDS-direct slots = fragment-read addresses", ok && (long)seen.size() == BK * TBN * 2 / 16);
    // staged epilogue: a wave's WTM x WTN tile, rows of CPRC chunks
    constexpr int CPRC = WTN / 8, RPI = 1024 / (WTN * 2);
    long ew = 0, ewn = 0, er = 0, ern = 0, old = 0;
    std::set<long> slots;
    for (int i = 0; i < FFM; ++i)
        for (int j = 0; j < FFN; ++j)
            for (int q = 0; q < 4; ++q) {
                std::vector<long> a(64), b(64);
                for (int l = 0; l < 64; ++l) {
                    const int row = 32 * i + (l & 31), half = l >> 5, L = 4 * j + q;
                    a[l] = 2L * (row * WTN + lds::h16_epi_write<CPRC>(row, L, half));
                    slots.insert(a[l]);
                    // the layout before: half flipped on the row bit above the chunk count
                    b[l] = 2L * (row * WTN + ((L ^ (row % CPRC)) << 3) + ((half ^ ((row / CPRC) & 1)) << 2));
                }
                ew += wr8(a); ++ewn; old += wr8(b);
            }
    placement(name, "epilogue staging: every 8-byte slot written once", (long)slots.size() == WTM * WTN / 4);
    bool rok = true;
    for (int it = 0; it < WTM / RPI; ++it) {
        std::vector<long> a(64);
        for (int l = 0; l < 64; ++l) {
            const int row = RPI * it + l / CPRC, cl = l % CPRC;
            a[l] = 2L * (row * WTN + lds::h16_epi_read<CPRC>(row, cl));
            // the chunk read back holds logical chunk cl, halves swapped when flagged
            const int sw = lds::h16_epi_swap(row);
            rok &= a[l] + 8 * sw == 2L * (row * WTN + lds::h16_epi_write<CPRC>(row, cl, 0)) &&
                   a[l] + 8 * (1 - sw) == 2L * (row * WTN + lds::h16_epi_write<CPRC>(row, cl, 1));
        }
        er += rd(a, 16); ++ern;
    }
    placement(name, "epilogue read-back finds each logical chunk", rok);
    report(name, "epilogue ds_write_b64", ewn, ew);
    report(name, "epilogue ds_read_b128", ern, er);
    report(name, "epilogue ds_write_b64, earlier layout (half flipped on row / chunks)", ewn, old);
}

// ------------------------------------------------------------------ fp8
template <int QB>
static void fp8(const char *name)
{
    // 8 waves: 256x256 tiles as 2 x 4 waves of 128 x 64; 128x128 as 4 x 2 of 32 x 64
    constexpr int WM = QB == 256 ? 2 : 4, WN = 8 / WM, WTM = QB / WM, WTN = QB / WN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    long ar = 0, ai = 0, br = 0, bi = 0;
    for (int wave = 0; wave < 8; ++wave) {
        const int wm0 = (wave / WN) * WTM, wn0 = (wave % WN) * WTN;
        for (int i = 0; i < FM; ++i)
            for (int c2 = 0; c2 < 2; ++c2) {                  // two ds_read_b128 per A tile
                std::vector<long> a(64);
                for (int l = 0; l < 64; ++l) a[l] = lds::fp8_a_frag(wm0 + 32 * i + (l & 31), 2 * (l >> 5) + c2);
                ar += rd(a, 16); ++ai;
            }
        for (int j = 0; j < FN; ++j)
            for (int q = 0; q < 4; ++q) {                     // four tr_b8 reads per B tile
                std::vector<long> a(64);
                for (int l = 0; l < 64; ++l) {
                    const int g = l >> 4, w16 = l & 15, r8 = w16 >> 1;
                    const int n = wn0 + 32 * j + 16 * (g & 1) + 8 * (w16 & 1);
                    const int krow = 32 * (g >> 1) + 8 * q + r8;
                    if (lds::fp8_b_col<QB>(r8, n) != lds::fp8_b_col<QB>(krow, n)) ++failures;
                    a[l] = (32 * (g >> 1) + r8) * QB + lds::fp8_b_col<QB>(r8, n) + 8 * q * QB;
                }
                br += rd(a, 8); ++bi;
            }
    }
    report(name, "main loop A ds_read_b128 (per K step of 64)", ai, ar);
    report(name, "main loop B ds_read_b64_tr_b8 (per K step of 64)", bi, br);
    bool ok = true;
    std::set<long> seen;
    for (int b = 0; b < QB * 64 / 1024; ++b)
        for (int l = 0; l < 64; ++l) {
            int row, chunk;
            lds::fp8_a_dma(b, l, row, chunk);
            const long slot = 1024L * b + 16 * l;
            ok &= slot == lds::fp8_a_frag(row, chunk) && seen.insert(slot).second;
        }
    placement(name, "A stage: LDS-direct slots = fragment-read addresses", ok && (long)seen.size() == QB * 64 / 16);
    ok = true; seen.clear();
    for (int b = 0; b < 64 * QB / 1024; ++b)
        for (int l = 0; l < 64; ++l) {
            int row, chunk;
            lds::fp8_b_dma<QB>(b, l, row, chunk);
            const long slot = 1024L * b + 16 * l;
            ok &= slot == row * QB + lds::fp8_b_col<QB>(row, 16 * chunk) && row < 64 && seen.insert(slot).second;
        }
    placement(name, "B stage: LDS-direct slots = fragment-read addresses", ok && (long)seen.size() == 64 * QB / 16);
    long ew = 0, ewn = 0, er = 0, ern = 0;
    std::set<long> slots;
    for (int i = 0; i < FM; ++i)
        for (int j = 0; j < FN; ++j)
            for (int q = 0; q < 4; ++q) {
                std::vector<long> a(64);
                for (int l = 0; l < 64; ++l) {
                    const int row = 32 * i + (l & 31);
                    a[l] = 2L * (row * WTN + lds::fp8_epi_write(row, 4 * j + q, l >> 5));
                    slots.insert(a[l]);
                }
                ew += wr8(a); ++ewn;
            }
    placement(name, "epilogue staging: every 8-byte slot written once", (long)slots.size() == WTM * WTN / 4);
    for (int it = 0; it < WTM / 8; ++it) {
        std::vector<long> a(64);
        for (int l = 0; l < 64; ++l) {
            const int row = 8 * it + (l >> 3);
            a[l] = 2L * (row * WTN + lds::fp8_epi_read(row, l & 7));
        }
        er += rd(a, 16); ++ern;
    }
    report(name, "epilogue ds_write_b64", ewn, ew);
    report(name, "epilogue ds_read_b128", ern, er);
}

// ----------------------------------------------------------------- fp32
static void f32(const char *name)
{
    long ar = 0, ai = 0, br = 0, bi = 0;
    for (int wave = 0; wave < 4; ++wave) {
        const int wm0 = (wave / 2) * 64, wn0 = (wave % 2) * 64;
        for (int s = 0; s < 2; ++s) {
            for (int i = 0; i < 2; ++i) {
                std::vector<long> a(64);
                for (int l = 0; l < 64; ++l) a[l] = 4L * lds::f32_a_frag(wm0 + 32 * i + (l & 31), 2 * s + (l >> 5));
                ar += rd(a, 16); ++ai;
            }
            for (int e = 0; e < 4; ++e)
                for (int j = 0; j < 2; ++j) {
                    std::vector<long> a(64);
                    for (int l = 0; l < 64; ++l)
                        a[l] = 4L * lds::f32_b_elem(8 * s + 4 * (l >> 5) + e, wn0 + 32 * j + (l & 31));
                    br += rd(a, 4); ++bi;
                }
        }
    }
    report(name, "main loop A ds_read_b128 (per K step of 16)", ai, ar);
    report(name, "main loop B ds_read_b32 (per K step of 16)", bi, br);
    bool ok = true;
    std::set<long> seen;
    for (int b = 0; b < 128 * 16 * 4 / 1024; ++b)
        for (int l = 0; l < 64; ++l) {
            int row, chunk;
            lds::f32_a_dma(b, l, row, chunk);
            const long slot = 1024L * b + 16 * l;
            ok &= slot == 4L * lds::f32_a_frag(row, chunk) && seen.insert(slot).second;
        }
    placement(name, "A stage: LDS-direct slots = fragment-read addresses", ok && seen.size() == 512);
    ok = true; seen.clear();
    for (int b = 0; b < 16 * 128 * 4 / 1024; ++b)
        for (int l = 0; l < 64; ++l) {
            int row, chunk;
            lds::f32_b_dma(b, l, row, chunk);
            const long slot = 1024L * b + 16 * l;
            ok &= slot == 4L * lds::f32_b_elem(row, 4 * chunk) && row < 16 && seen.insert(slot).second;
        }
    placement(name, "B stage: LDS-direct slots = fragment-read addresses", ok && seen.size() == 512);
}

// Without the swizzles (chunk index = logical chunk) the same reads conflict:
// the checks below are not vacuous.
static void unswizzled()
{
    long ar = 0, br = 0;
    for (int i = 0; i < 4; ++i) {
        std::vector<long> a(64);
        for (int l = 0; l < 64; ++l) a[l] = 2L * ((32 * i + (l & 31)) * 32 + ((l >> 5) << 3));
        ar += rd(a, 16);
    }
    for (int j = 0; j < 4; ++j) {
        std::vector<long> a(64);
        for (int l = 0; l < 64; ++l) {
            const int g = l >> 4, w16 = l & 15, r4 = w16 >> 2, c4 = w16 & 3;
            a[l] = 2L * ((8 * (g >> 1) + r4) * 256 + 32 * j + 16 * (g & 1) + 4 * c4);
        }
        br += rd(a, 8);
    }
    report("bf16 256x256 without swizzles", "A ds_read_b128 x4 / B tr_b16 x4", 8, ar * 1000 + br);
}

int main()
{
    h16<256, 256>("bf16/fp16 256x256");
    h16<128, 128>("bf16/fp16 128x128");
    h16<128, 256>("bf16/fp16 128x256");
    fp8<256>("fp8 256x256");
    fp8<128>("fp8 128x128");
    f32("fp32 128x128");
    unswizzled();
    printf("FAILURES %d\n", failures);
    return 0;
}
"""


@pytest.fixture(scope="module")
def lines():
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "banks.hip"), os.path.join(d, "banks")
        open(src, "w").write(HARNESS)
        r = subprocess.run(["/opt/rocm/bin/hipcc", "-O1", "-std=c++17", "-I", CSRC,
                            "-I", os.path.join(ROOT, "include"), src, "-o", exe],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        out = subprocess.run([exe], capture_output=True, text=True, timeout=120)
        assert out.returncode == 0, out.stderr
        return out.stdout.splitlines()


def _banks(lines):
    rows = {}
    for ln in lines:
        if ln.startswith("BANKS "):
            kernel, what, n, extra = [p.strip() for p in ln[6:].split("|")]
            rows[(kernel, what)] = (int(n.split()[-1]), int(extra.split()[-1]))
    return rows


def test_placement_lds_direct_writes_match_fragment_reads(lines):
    bad = [ln for ln in lines if ln.startswith("PLACE ") and not ln.endswith("ok")]
    assert not bad, bad
    assert sum(ln.startswith("PLACE ") for ln in lines) == 3 * 4 + 2 * 3 + 2   # every kernel checked
    assert lines[-1] == "FAILURES 0"


def test_main_loops_and_epilogues_conflict_free(lines):
    rows = _banks(lines)
    checked = [(k, w) for (k, w) in rows if "earlier layout" not in w and "without" not in k]
    assert len(checked) == 3 * 4 + 2 * 4 + 2
    for key in checked:
        assert rows[key][1] == 0, f"{key}: {rows[key][1]} extra cycles"


def test_model_reproduces_the_measured_conflict_count(lines):
    """The earlier epilogue layout of the 256x256 bf16 kernel costs 256 extra
    cycles per wave in the model: 262144 per launch over 1024 waves, the count
    SQ_LDS_BANK_CONFLICT read on MI355X for that kernel (and 0 for its loop)."""
    rows = _banks(lines)
    n, old = rows[("bf16/fp16 256x256", "epilogue ds_write_b64, earlier layout (half flipped on row / chunks)")]
    assert n == 64 and old == 256
    assert old * 1024 == 262144
    # 64-wide wave tiles (128x128) always flipped on row bit 3: no change there
    assert rows[("bf16/fp16 128x128", "epilogue ds_write_b64, earlier layout (half flipped on row / chunks)")][1] == 0


def test_swizzles_are_what_makes_the_reads_conflict_free(lines):
    rows = _banks(lines)
    _, code = rows[("bf16 256x256 without swizzles", "A ds_read_b128 x4 / B tr_b16 x4")]
    a_extra, b_extra = divmod(code, 1000)
    assert a_extra > 0 and b_extra > 0
