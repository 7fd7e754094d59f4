"""The library's E4M3 encoder / decoder (csrc/common.h, host-callable) against
the oracle's, on the CPU: every binary32 value in [-448.5, 448.5] with its top
20 bits varied and 5 low-bit patterns (ties and their neighbours included), and
every finite code.  (The GPU tests check the quantiser's codes, which use the
hardware conversion, against the oracle at full size.)"""
import os
import subprocess
import tempfile

import pytest

import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = r'''
#include "w8a8_quantized_amd/csrc/common.h"
#include <cstdio>
#include <cstring>
#include <dlfcn.h>
int main(int argc, char** argv) {
  void* h = dlopen(argv[1], RTLD_NOW);
  if (!h) return 2;
  auto enc = (uint8_t(*)(float))dlsym(h, "sqo_e4m3_encode");
  auto dec = (float(*)(uint8_t))dlsym(h, "sqo_e4m3_decode");
  long bad = 0, n = 0;
  for (uint32_t hi = 0; hi < (1u << 20); ++hi)
    for (uint32_t lo : {0u, 1u, 0x7FFu, 0x800u, 0xFFFu}) {
      uint32_t bits = (hi << 12) | lo;
      float v; memcpy(&v, &bits, 4);
      if (!(v == v) || __builtin_fabsf(v) > 448.5f) continue;
      ++n;
      bad += sq::e4m3_code(v) != enc(v);
    }
  for (int c = 0; c < 256; ++c) {
    if ((c & 0x7F) == 0x7F) continue;
    float a = sq::e4m3_value(c), b = dec((uint8_t)c);
    bad += memcmp(&a, &b, 4) != 0;
  }
  printf("%ld %ld\n", n, bad);
  return bad != 0;
}
'''


def test_library_e4m3_codec_matches_oracle():
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    lib = O.sq_oracle.build()
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "codec.cpp"), os.path.join(d, "codec")
        open(src, "w").write(SRC)
        subprocess.run([hipcc, "-x", "hip", "--offload-arch=gfx950", "-O2", "-std=c++17", "-ffp-contract=off",
                        "-I", ROOT, src, "-o", exe, "-ldl"], check=True, capture_output=True)
        r = subprocess.run([exe, lib], capture_output=True, text=True)
    n, bad = map(int, r.stdout.split())
    assert n > 2_700_000 and bad == 0, r.stdout
