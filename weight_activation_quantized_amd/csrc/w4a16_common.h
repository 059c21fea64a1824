// 4-bit weight unpacking into MFMA B-operand fragments (gfx950).
//
// Weight layout (LMDeploy toolkit overview, section 2.5: 4-bit weights in
// groups of G = 128 input channels; LMDeploy 4-bit deployment guide, section
// 3.2: G = 64 for the vision tower; the pages give no bit layout, so field j
// of word c, least significant first, is column 8c+j): qweight[K, N/8]
// int32, scales[K/G, N] fp16, qzeros[K/G, N/8] int32 packed like qweight.
//
// The packing runs along N while an MFMA B fragment wants 8 consecutive k of
// one column in one lane. A lane therefore loads one word from each of 8
// consecutive rows of the same packed column and transposes in registers:
// for each row pair it gathers matching bytes of the two words with one
// v_perm_b32, then each 4-bit field becomes an fp16 by OR-ing it into the
// mantissa of 1024.0. Fields in bits 0-3 of a byte give 1024 + q, fields in
// bits 4-7 give 1024 + 16q (no shift needed); the odd-field fragments carry
// a factor 16 that is removed with the scale. Subtracting the zero point as
// (1024 + z) or (1024 + 16z) is exact in fp16, so a fragment holds q - z (or
// 16(q - z)) exactly.
#pragma once

#include "device_common.h"

namespace mq {

// The two field masks and the 1024.0 pattern, held in VGPRs: gfx9 VOP3
// encodings take no literal constants, so with literal masks the compiler
// splits each (v & mask) | magic into v_and_b32 + v_or_b32; with register
// operands it emits one v_and_or_b32 (a third fewer VALU ops in the unpack).
// The values come from non-volatile asm the compiler can hoist out of loops.
// magic64 is the pattern of 64.0 (0x5400): a field in bits 4-7 OR-ed into
// it reads 64 + q (the mantissa step at 64 is 1/16), for kernels that
// scale the fragments in fp16 and so need the high field without the
// factor 16.
// bmagic is the bf16 pattern of 128.0 (0x4300): a field in bits 0-3 OR-ed
// into it reads 128 + q exactly (bf16 keeps 8 significant bits), the bf16
// counterpart of 1024 + q. A bf16 exponent starts at bit 7, so a field in
// bits 4-7 is first shifted down.
struct NibConst {
  uint32_t lo, hi, magic, magic64, bmagic;
};
__device__ __forceinline__ NibConst nib_const() {
  NibConst c;
  asm("v_mov_b32 %0, 0x000f000f" : "=v"(c.lo));
  asm("v_mov_b32 %0, 0x00f000f0" : "=v"(c.hi));
  asm("v_mov_b32 %0, 0x64006400" : "=v"(c.magic));
  asm("v_mov_b32 %0, 0x54005400" : "=v"(c.magic64));
  asm("v_mov_b32 %0, 0x43004300" : "=v"(c.bmagic));
  return c;
}

// A fragment of eight 1.0 values (fp16 0x3C00 or bf16 0x3F80), for the MFMA
// that sums x over a group.
template <bool kBf16>
__device__ __forceinline__ f16x8 ones_fragment() {
  const uint32_t one2 = kBf16 ? 0x3F803F80u : 0x3C003C00u;
  return __builtin_bit_cast(f16x8, u32x4{one2, one2, one2, one2});
}

// -(1024 + z_p) (even p) or -(1024 + 16 z_p) (odd p), replicated in both
// fp16 halves, for the 8 fields of zero-point word zw.
__device__ __forceinline__ void zero_bias(uint32_t zw, uint32_t (&negz)[8]) {
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const uint32_t e = (p & 1) ? (((zw >> (4 * (p - 1))) & 0xF0u) | 0xE400u)
                               : (((zw >> (4 * p)) & 0x0Fu) | 0xE400u);
    negz[p] = e | (e << 16);
  }
}

// Fragments of (q - z), or 16 (q - z) for odd p, for one 32-row k-step.
// w[e] is the word of row 8h + e; b[p][e] belongs to field p of row 8h + e.
__device__ __forceinline__ void unpack_step(const uint32_t (&w)[8], const uint32_t (&negz)[8],
                                            f16x8 (&b)[8]) {
  const NibConst c = nib_const();
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const uint32_t lo = byte_perm(w[2 * t + 1], w[2 * t], 0x05040100u);  // bytes 0,1 of both rows
    const uint32_t hi = byte_perm(w[2 * t + 1], w[2 * t], 0x07060302u);  // bytes 2,3 of both rows
    const uint32_t lo8 = lo >> 8, hi8 = hi >> 8;
    const uint32_t v[8] = {(lo & c.lo) | c.magic,  (lo & c.hi) | c.magic,  (lo8 & c.lo) | c.magic,
                           (lo8 & c.hi) | c.magic, (hi & c.lo) | c.magic,  (hi & c.hi) | c.magic,
                           (hi8 & c.lo) | c.magic, (hi8 & c.hi) | c.magic};
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const f16x2 d = as_f16x2(v[p]) + as_f16x2(negz[p]);
      b[p][2 * t] = d[0];
      b[p][2 * t + 1] = d[1];
    }
  }
}

}  // namespace mq
