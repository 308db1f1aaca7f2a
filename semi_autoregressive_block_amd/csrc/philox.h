// Philox4x32-10 counter-based generator and the Gumbel draw built on it.
//
// Philox is defined in Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers:
// As Easy as 1, 2, 3" (SC'11), Section 4.2: ten rounds over four 32-bit
// counter words; each round forms the two 64-bit products of words 0 and 2
// with fixed odd multipliers, XORs their high halves with the other two
// words and the round key, and permutes; the round key advances by a Weyl
// increment between rounds.  The multiply is done as one 32x32->64 product
// per word (v_mad_u64_u32 on gfx950).
//
// Gumbel noise for vocabulary index v of (row, step): x = word (v & 3) of the
// block at counter (v >> 2, step, row, 0) under key (seed_lo, seed_hi);
// u = ((x >> 9) + 1/2) * 2^-23, exact in float32 and inside [2^-24, 1-2^-24];
// E = -ln u, G = -ln E.
#pragma once

#include "common.h"

namespace dspark {

__device__ __forceinline__ u32x4 philox4x32_10(u32x4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c.x;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c.z;
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    c = u32x4{hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0};
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

// Gumbel(0,1) from one raw 32-bit draw.  E = -ln u must keep a small
// RELATIVE error (G = -ln E amplifies it) also for u close to 1, where
// ln u suffers cancellation; there E is taken from w = 1 - u (exact) with
// the series w + w^2/2 + w^3/3 + w^4/4 + w^5/5 (truncation below 2^-25
// relative for w < 2^-5).
__device__ __forceinline__ float gumbel_from_bits(uint32_t x) {
  constexpr float kLn2 = 0.69314718055994531f;
  const float u = ((float)(x >> 9) + 0.5f) * 0x1.0p-23f;
  const float w = 1.0f - u;  // exact (Sterbenz) for u >= 1/2
  const float series = w * fmaf(w, fmaf(w, fmaf(w, fmaf(w, 0.2f, 0.25f), 1.0f / 3.0f), 0.5f), 1.0f);
  const float viaLog = -kLn2 * __builtin_amdgcn_logf(u);
  const float E = (w < 0.03125f) ? series : viaLog;
  return -kLn2 * __builtin_amdgcn_logf(E);
}

}  // namespace dspark
