"""CPU check of the hybrid FFN's LDS layout (ffn_lds.h, the arithmetic the
kernels in ffn.hip use for their LDS offsets): over every shape the host
accepts (E 64..8192, rank 64..4096, hidden up to 2^20, all multiples of 64),
each launch's staged codes, group scales, wavefront partials and reduced
outputs end inside the static LDS instance the host picks for it, and that
instance fits a gfx950 work-group's 160 KB."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "latent_kv_attention_lr_amd", "csrc")

PROGRAM = r"""
#include <algorithm>
#include <cstdio>
#include "ffn_lds.h"
using namespace lr::ffnlds;
int main() {
  long bad = 0, checked = 0;
  auto need = [&](bool ok, const char* what, int v) { ++checked; if (!ok) { if (bad < 5) std::printf("%s %d\n", what, v); ++bad; } };
  for (int E = 64; E <= 8192; E += 64) {            // k_ffn_in: one block of E columns
    const int lds = instance_for(in_extent(E));
    need(lds != 0 && in_extent(E) <= lds && lds <= kLdsLimit, "in", E);
    need(block_bytes(E) <= code_area(block_bytes(E)) && red_bytes(4) <= code_area(block_bytes(E)), "in area", E);
  }
  for (int r = 64; r <= 4096; r += 64) {            // k_ffn_mid: two blocks of r columns
    const int lds = instance_for(mid_extent(r));
    need(lds != 0 && mid_extent(r) <= lds && lds <= kLdsLimit, "mid", r);
    need(2 * block_bytes(r) <= code_area(2 * block_bytes(r)), "mid area", r);
  }
  for (int Fp = 64; Fp <= (1 << 20); Fp += 64) {    // k_ffn_out: chunks of the hidden dimension
    const OutShape s = out_shape(Fp);
    const int kc = std::min(s.chunk, Fp);
    need(out_extent(kc, s.rt) <= s.lds && out_extent(s.chunk, s.rt) <= s.lds && s.lds <= kLdsLimit, "out", Fp);
    need(red_bytes(s.rt) <= code_area(block_bytes(kc)) && s.rt <= 2, "out area", Fp);
    for (int k0 = 0; k0 < Fp; k0 += s.chunk) {        // every chunk's block fits the first one's area
      const int kn = std::min(s.chunk, Fp - k0);
      if (kn != kc) need(block_bytes(kn) <= code_area(block_bytes(kc)), "out chunk", Fp);
    }
  }
  std::printf("checked %ld, failed %ld\n", checked, bad);
  return bad != 0;
}
"""


def test_every_ffn_lds_offset_fits_its_instance(tmp_path):
    src = tmp_path / "ffn_lds_check.cpp"
    exe = tmp_path / "ffn_lds_check"
    src.write_text(PROGRAM)
    subprocess.run(["g++", "-std=c++17", "-O1", "-I", CSRC, str(src), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout
    assert "failed 0" in r.stdout
