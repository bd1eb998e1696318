"""CPU replay of the fp32 quotient the bf16 decode kernel uses for f(j).

Inside a block of 16 keys starting at j0 = q0 * G + r0 the kernel forms
f(j0 + col) = floor((j0 + col) / G) (eq. f, "Dynamic Bifocal RoPE") as
q0 + trunc((float(r0 + col) + 0.5f) * (1.f / G)) in fp32, for G < 2^20.
This test compiles the same fp32 expression in plain C (IEEE single, round
to nearest even, no contraction) and compares it with the integer quotient
n // G for every n = r0 + col in [0, G + 15): exhaustively for G < 2^16 and
for 3000 seeded G up to 2^20 at every n near 0, near G and 2000 random n.
It also replays the expression with the reciprocal one ulp above and one ulp
below its correctly rounded value, so the result does not hinge on how the
device rounds 1/G.  The device code itself is compared bit-exactly by the
GPU test of jl_bifocal_decode_key_rows.
"""
import os
import shutil
import subprocess
import tempfile

import pytest

C_SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

static uint64_t state = 0x853c49e6748fea9bULL;
static uint32_t next_u32(void) {  /* xorshift64* */
  state ^= state >> 12; state ^= state << 25; state ^= state >> 27;
  return (uint32_t)((state * 0x2545F4914F6CDD1DULL) >> 32);
}

static long bad = 0, checked = 0;

static void check(int G, long n, float inv) {
  volatile float x = (float)n + 0.5f;
  volatile float y = x * inv;
  const long got = (long)(int)y;
  ++checked;
  if (got != n / G) {
    if (bad < 10) fprintf(stderr, "G=%d n=%ld got %ld want %ld\n", G, n, got, n / G);
    ++bad;
  }
}

static void check_all_inv(int G, long n) {
  const float inv = 1.f / (float)G;
  check(G, n, inv);
  check(G, n, nextafterf(inv, 2.f));
  check(G, n, nextafterf(inv, 0.f));
}

int main(int argc, char** argv) {
  const int gex = atoi(argv[1]);      /* exhaustive below this G */
  const int nsamp = atoi(argv[2]);    /* sampled G in [gex, 2^20) */
  for (int G = 1; G < gex; ++G)
    for (long n = 0; n < (long)G + 15; ++n) check_all_inv(G, n);
  for (int s = 0; s < nsamp; ++s) {
    const int G = gex + (int)(next_u32() % (uint32_t)((1 << 20) - gex));
    for (long n = 0; n < 32; ++n) check_all_inv(G, n);
    for (long n = G - 32; n < (long)G + 15; ++n) if (n >= 0) check_all_inv(G, n);
    for (int r = 0; r < 2000; ++r) check_all_inv(G, (long)(next_u32() % (uint32_t)(G + 15)));
  }
  printf("%ld %ld\n", checked, bad);
  return bad != 0;
}
"""


def _gcc():
    cc = shutil.which("gcc") or shutil.which("cc")
    if not cc:
        pytest.skip("no C compiler")
    return cc


def test_decode_fp32_quotient_exact():
    cc = _gcc()
    with tempfile.TemporaryDirectory() as td:
        src = os.path.join(td, "replay.c")
        exe = os.path.join(td, "replay")
        with open(src, "w") as f:
            f.write(C_SRC)
        subprocess.run([cc, "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-msse2", "-mfpmath=sse",
                        src, "-o", exe, "-lm"], check=True)
        r = subprocess.run([exe, str(1 << 16), "3000"], capture_output=True, text=True, timeout=600)
    checked, bad = (int(x) for x in r.stdout.split())
    assert checked > 6_000_000_000, checked
    assert r.returncode == 0 and bad == 0, r.stderr


def test_replay_detects_a_wrong_quotient():
    """The replay is able to fail: without the +0.5 offset the truncated
    product is below the integer at n = G (1/G rounded down)."""
    cc = _gcc()
    src_bad = C_SRC.replace("(float)n + 0.5f", "(float)n + 0.0f")
    with tempfile.TemporaryDirectory() as td:
        src = os.path.join(td, "replay.c")
        exe = os.path.join(td, "replay")
        with open(src, "w") as f:
            f.write(src_bad)
        subprocess.run([cc, "-O2", "-std=c99", "-ffp-contract=off", src, "-o", exe, "-lm"], check=True)
        r = subprocess.run([exe, "4096", "10"], capture_output=True, text=True, timeout=600)
    assert r.returncode != 0
