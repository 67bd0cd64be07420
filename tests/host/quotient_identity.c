/* Host check of the write kernels' division-free quotient (kv4_write.hip,
 * `quotient`): for every bf16 absmax a (taken with a stride given on the
 * command line), scale = fl(a / qmax) in [2^-100, 2^100], r = fl(1 / scale),
 * and every bf16 y with |y| <= a (both signs), the codes taken from
 *   q0 = fl(y r), e = fma(-q0, scale, y), q = fma(e, r, q0)
 * equal the codes taken from the IEEE quotient fl(y / scale): rint for qmax 7
 * and 127, the e4m3fn byte (quotient of |y|, sign of y) for 448. Prints the
 * number of pairs and of mismatches; exits 1 on any mismatch. Compile without
 * fast-math and without fp contraction. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* nearest-even e4m3fn byte of q, saturating at 448, sign bit of q */
static uint32_t e4m3(float q) {
  const uint32_t u = u_of(q), sign = (u >> 24) & 0x80u, a = u & 0x7FFFFFFFu;
  uint32_t code;
  if (a >= 0x43E00000u) {
    code = 0x7Eu;
  } else if (a < 0x3C800000u) {
    code = (uint32_t)rintf(f_of(a) * 512.0f);
  } else {
    uint32_t bits = a >> 20;
    const uint32_t rem = a & 0xFFFFFu;
    bits += (rem > 0x80000u || (rem == 0x80000u && (bits & 1u))) ? 1u : 0u;
    code = bits - (120u << 3);
    if (code > 0x7Eu) code = 0x7Eu;
  }
  return code | sign;
}

int main(int argc, char** argv) {
  const uint32_t stride = argc > 1 ? (uint32_t)strtoul(argv[1], NULL, 10) : 1u;
  const float qmax[3] = {7.0f, 127.0f, 448.0f};
  uint64_t pairs = 0, bad = 0;
  for (int iq = 0; iq < 3; ++iq) {
    for (uint32_t ua = 1; ua < 0x7F80u; ua += stride) {
      const float amax = f_of(ua << 16);
      const float scale = amax / qmax[iq];
      if (!(scale >= 0x1p-100f) || !(scale <= 0x1p100f)) continue;
      const float r = 1.0f / scale;
      for (uint32_t uy = 0; uy <= ua; ++uy) {
        for (uint32_t sg = 0; sg < 2; ++sg) {
          const float y = f_of((uy << 16) | (sg << 31));
          const float want = y / scale;
          int ok;
          if (iq < 2) {
            const float q0 = y * r, e = fmaf(-q0, scale, y), q = fmaf(e, r, q0);
            ok = rintf(q) == rintf(want);
          } else {
            const float ya = fabsf(y), q0 = ya * r, e = fmaf(-q0, scale, ya), qa = fmaf(e, r, q0);
            ok = e4m3(f_of(u_of(qa) | (u_of(y) & 0x80000000u))) == e4m3(want);
          }
          ++pairs;
          if (!ok) {
            if (bad < 10) printf("mismatch: qmax %g amax %a y %a\n", qmax[iq], amax, y);
            ++bad;
          }
        }
      }
    }
  }
  printf("pairs %llu mismatches %llu\n", (unsigned long long)pairs, (unsigned long long)bad);
  return bad != 0;
}
