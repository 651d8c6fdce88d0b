// fp8_e4m3_block64 quantization of one bf16 row by one wave (the CSA CPU
// page's `finalize_attention_record` pack loop): the quantize-on-append
// kernel and the shared-latent forward kernel's in-launch append both use it,
// so the two produce the same bytes.
#pragma once

#include "sa_internal.h"

namespace sa {

// E4M3FN code of x * 2^(127 - e), x given by its fp32 bits: round to nearest
// even, saturate at 448 (code 0x7E), sign kept (a negative value that rounds
// to zero gives 0x80). Integer-exact: x = sig * 2^ex, and the quantum of the
// target binade is 2^q with q = max(floor(log2 v), -6) - 3 (the subnormal
// quantum 2^-9 below 2^-6). The code bits are (max(lg,-6)+7)*8 + n - 8, which
// runs continuously across the subnormal/normal seam and binade carries.
__device__ __forceinline__ uint32_t e4m3fn_encode_scaled(uint32_t w, int e) {
  const uint32_t sign = (w >> 31) << 7;
  const uint32_t a = w & 0x7fffffffu;
  if (a == 0) return sign;
  const int E = (int)(a >> 23);
  const uint32_t sig = E ? ((a & 0x7fffffu) | 0x800000u) : (a & 0x7fffffu);
  const int ex = (E ? E - 150 : -149) + 127 - e;
  const int lg = (31 - __clz((int)sig)) + ex;
  const int lgc = lg < -6 ? -6 : lg;
  const int shift = (lgc - 3) - ex;
  uint32_t n;
  if (shift <= 0) {
    n = sig << (-shift);
  } else if (shift >= 32) {
    n = 0;
  } else {
    n = sig >> shift;
    const uint32_t rem = sig & ((1u << shift) - 1u);
    const uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (n & 1u))) n += 1u;
  }
  int code = ((lgc + 7) << 3) + (int)n - 8;
  if (code > 0x7e) code = 0x7e;
  return sign | (uint32_t)code;
}

// Maximum over the 64 lanes, all on the VALU: DPP within rows of 16 lanes,
// then the gfx950 permlane swaps across rows.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xb1, 0xf, 0xf, false));   // quad_perm 1,0,3,2
  x = max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4e, 0xf, 0xf, false));   // quad_perm 2,3,0,1
  x = max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x124, 0xf, 0xf, false));  // row_ror 4
  x = max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x128, 0xf, 0xf, false));  // row_ror 8
  const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = max(a[0], a[1]);
  const auto c = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return max(c[0], c[1]);
}

// Quantize the bf16 row src (dk <= 1024 values, the last `rope` of them kept
// as little-endian BF16) into the record at dst, by the 64 lanes of one wave:
// lane l owns element l of every 64-value block. Per block the E8M0 scale
// byte is floor(log2 amax) - 8 + 127 clamped to [0, 254] (127 and zero codes
// for an all-zero block) and the codes are E4M3FN of x * 2^(127 - e). A row
// holding a NaN or an infinity is left unwritten; returns true for it.
__device__ __forceinline__ bool quantize_row_wave(const uint16_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                  int dk, int rope, int lane) {
  // the whole row first, every load in flight at once (dk <= 64 * MAXV)
  constexpr int MAXV = 16;
  uint32_t vals[MAXV];
#pragma unroll
  for (int k = 0; k < MAXV; k++) vals[k] = 64 * k + lane < dk ? src[64 * k + lane] : 0u;
  bool bad = false;
#pragma unroll
  for (int k = 0; k < MAXV; k++) bad |= (vals[k] & 0x7f80u) == 0x7f80u;
  if (__ballot(bad) != 0ull) return true;
  const int nblk = (dk - rope) / 64;
#pragma unroll
  for (int j = 0; j < MAXV; j++) {
    if (j >= nblk) break;
    const uint32_t w = vals[j] << 16;
    const uint32_t amax = wave_max_u32(w & 0x7fffffffu);
    uint32_t code = 0;
    int e = 127;
    if (amax != 0) {
      const int E = (int)(amax >> 23);
      const int k = E ? E - 127 : (31 - __clz((int)(amax & 0x7fffffu))) - 149;
      e = k - 8 + 127;
      e = e < 0 ? 0 : (e > 254 ? 254 : e);
      code = e4m3fn_encode_scaled(w, e);
    }
    if (lane == 0) dst[65 * j] = (uint8_t)e;
    dst[65 * j + 1 + lane] = (uint8_t)code;
  }
  // the RoPE tail: element dk - rope + i is vals[nblk + i / 64] of lane i % 64
  uint8_t* tail = dst + 65 * nblk;
#pragma unroll
  for (int m = 0; m < MAXV; m++) {
    const int i = 64 * m + lane;
    if (nblk + m < MAXV && i < rope) {
      const uint32_t bits = vals[nblk + m < MAXV ? nblk + m : 0];
      tail[2 * i] = (uint8_t)(bits & 0xff);
      tail[2 * i + 1] = (uint8_t)(bits >> 8);
    }
  }
  return false;
}

// E4M3FN code c times 2^(e - 127) as bf16 bits, exact where representable
// (round to nearest even otherwise); the NaN code and scale byte 255 give NaN.
__device__ __forceinline__ uint32_t fp8_code_to_bf16_exact(uint32_t c, uint32_t e) {
  const uint32_t mag = c & 0x7fu;
  if (mag == 0x7fu || e == 255u) return 0x7fc0u;
  const uint32_t E = mag >> 3, M = mag & 7u;
  float v = E ? __uint_as_float(((E + 120u) << 23) | (M << 20)) : (float)M * 0.001953125f;
  v = ldexpf(v, (int)e - 127);
  return (uint32_t)f32_to_bf16_rne(v) | ((c & 0x80u) << 8);
}

// E4M3FN decode of one packed word of four codes at block scale byte e into
// two words of bf16 pairs (codes 0,1 -> lo; 2,3 -> hi). For scale bytes
// 10..246 v_cvt_scalef32_pk_bf16_fp8 is exact (every code times 2^(e-127) is a
// bf16 normal); other bytes take the integer path above.
__device__ __forceinline__ void fp8x4_to_bf16x4(uint32_t cw, uint32_t e, uint32_t& lo, uint32_t& hi) {
  if (e >= 10u && e <= 246u) {
    const float s = __uint_as_float(e << 23);
    lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw, s, false));
    hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw, s, true));
  } else {
    lo = fp8_code_to_bf16_exact(cw & 0xffu, e) | (fp8_code_to_bf16_exact((cw >> 8) & 0xffu, e) << 16);
    hi = fp8_code_to_bf16_exact((cw >> 16) & 0xffu, e) | (fp8_code_to_bf16_exact(cw >> 24, e) << 16);
  }
}

}  // namespace sa
