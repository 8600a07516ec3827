// Host build of the device E4M3 quantizer's arithmetic (block_scaled_fp4_pre_amd/csrc/e4m3.h),
// for an exhaustive comparison with the oracle on the CPU.  Reads groups of 32 fp32
// values from stdin; writes per group 32 code bytes and the scale byte.
#define __host__
#define __device__
#include <stdio.h>
#include "../block_scaled_fp4_pre_amd/csrc/e4m3.h"

int main() {
  float v[32];
  unsigned char out[33];
  while (fread(v, sizeof(float), 32, stdin) == 32) {
    uint32_t amax = 0;
    for (int i = 0; i < 32; ++i) {
      const uint32_t a = moe::e4m3_f32_bits(v[i]) & 0x7FFFFFFFu;
      amax = a > amax ? a : amax;
    }
    const int e = moe::mx8_scale_exp(amax);
    const float inv = moe::e4m3_exp2(-e);
    for (int i = 0; i < 32; ++i) out[i] = (unsigned char)moe::e4m3_code(v[i] * inv);
    out[32] = (unsigned char)(e + 127);
    fwrite(out, 1, 33, stdout);
  }
  return 0;
}
