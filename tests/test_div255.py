"""The kernels write a quantized output as fl(fl(acc) * s_c) / 255 rounded to nearest even
(BinaryAttention section 2.4: A_q carries the scale 1/255).  They form the quotient in
three operations (the product with fl(1/255), the exact remainder by fma, one fma
correction; had_device.hpp div255_rn) instead of an IEEE division.  This checks that the
identity equals IEEE division on the host, over a strided sweep of all positive finite
float32 bit patterns plus denormals, powers of two and the largest values (a full
sweep of every pattern takes about half a minute on eight cores and also finds no
difference)."""
import ctypes
import shutil
import subprocess

import pytest

SRC = r"""
#include <math.h>
#include <stdint.h>
#include <string.h>
static float div255_rn(float x) {
  const float y = 1.0f / 255.0f;
  const float q0 = x * y;
  const float r = fmaf(-q0, 255.0f, x);
  return fmaf(r, y, q0);
}
static int check(uint32_t b) {
  float x, q;
  memcpy(&x, &b, 4);
  volatile float ref = x / 255.0f;
  q = div255_rn(x);
  if (q != ref) return 1;
  q = div255_rn(-x);
  return q != -ref;
}
long sweep(uint32_t stride) {
  long bad = 0;
  for (uint64_t u = 0; u < 0x7f800000ull; u += stride) bad += check((uint32_t)u);
  for (uint32_t u = 0; u < 0x00100000u; ++u) bad += check(u);            /* denormals */
  for (uint32_t u = 0x7f700000u; u < 0x7f800000u; ++u) bad += check(u);  /* largest values */
  for (uint32_t e = 1; e < 255; ++e)
    for (int d = -2; d <= 2; ++d) bad += check((e << 23) + (uint32_t)(d + 2));  /* near powers of two */
  return bad;
}
"""


@pytest.fixture(scope="module")
def lib(tmp_path_factory):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    d = tmp_path_factory.mktemp("div255")
    (d / "div255.c").write_text(SRC)
    so = d / "libdiv255.so"
    subprocess.run([gcc, "-O2", "-ffp-contract=off", "-shared", "-fPIC", "-o", str(so), str(d / "div255.c"), "-lm"],
                   check=True)
    lib = ctypes.CDLL(str(so))
    lib.sweep.argtypes = [ctypes.c_uint32]
    lib.sweep.restype = ctypes.c_long
    return lib


def test_div255_identity_matches_ieee_division(lib):
    assert lib.sweep(997) == 0


def test_div255_sweep_catches_a_wrong_reciprocal(tmp_path):
    # the same sweep with the correction step dropped (q0 alone) must find differences
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    src = SRC.replace("return fmaf(r, y, q0);", "(void)r; return q0;")
    (tmp_path / "bad.c").write_text(src)
    so = tmp_path / "libbad.so"
    subprocess.run([gcc, "-O2", "-ffp-contract=off", "-shared", "-fPIC", "-o", str(so), str(tmp_path / "bad.c"), "-lm"],
                   check=True)
    bad = ctypes.CDLL(str(so))
    bad.sweep.argtypes = [ctypes.c_uint32]
    bad.sweep.restype = ctypes.c_long
    assert bad.sweep(99991) > 0
