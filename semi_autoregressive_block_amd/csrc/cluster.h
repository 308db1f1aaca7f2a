// Device helpers of the cluster kernels: a row too long for one workgroup's
// registers is split over G co-resident workgroups (a cluster) that trade a
// few bytes of per-slice statistics through global memory.

#pragma once

#include <stdlib.h>

#include <algorithm>

#include "common.h"
#include "host_cache.h"

namespace dspark {
namespace cluster {

constexpr float kLog2e = 1.4426950408889634f;
constexpr unsigned kSpinLimit = 1u << 20;  // default poll bound of a wait (well under a second)
constexpr int kRsrcWord3 = 0x00020000;      // raw 32-bit buffer data format (gfx9 family)
constexpr int kNonTemporal = 2;             // streaming loads

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
// IEEE-754-2019 maximum (NaN-propagating): one v_maximum3 on gfx950, with no
// operand canonicalisation.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// ---- wave reductions: DPP inside each row of 16 lanes, then the four row
// results through scalar registers.  Every lane returns the same value, and
// the combination order is fixed, so equal inputs give equal bits anywhere.
__device__ __forceinline__ float lane_value(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ float uniform(float v) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}
__device__ __forceinline__ float wave_max(float v) {
  v = vmax(v, dpp_f32<kDppQuadSwap1>(v));
  v = vmax(v, dpp_f32<kDppQuadSwap2>(v));
  v = vmax(v, dpp_f32<kDppHalfMirror>(v));
  v = vmax(v, dpp_f32<kDppRowMirror>(v));
  return vmax(vmax(lane_value(v, 0), lane_value(v, 16)), vmax(lane_value(v, 32), lane_value(v, 48)));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f32<kDppQuadSwap1>(v);
  v += dpp_f32<kDppQuadSwap2>(v);
  v += dpp_f32<kDppHalfMirror>(v);
  v += dpp_f32<kDppRowMirror>(v);
  return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}

// ---- cluster exchange without fences.  A member publishes the four floats
// of a row's slice statistics as one 16-byte word (two 64-bit relaxed
// agent-scope atomic stores), and readers fetch it with two 64-bit relaxed
// agent-scope atomic loads; these bypass the per-XCD, mutually incoherent
// L2s and, unlike volatile accesses, make the wave wait for nothing until
// the value is used.  Every 32-bit lane of the word is single-copy atomic
// and carries a one-bit tag in its lowest mantissa bit, so a reader accepts
// the word only when all four tags equal the tag of the epoch it waits for.
// The slots alternate between two parities, so a slot awaited for epoch e
// holds either epoch e, epoch e - 2 or (first use) the zeros of the launch;
// the tag ((e + 1) >> 1) & 1 tells e from both, so no fence or per-poll
// cache maintenance is needed.  Dropping one mantissa bit changes a value
// by at most one unit in its last place.
__device__ __forceinline__ uint32_t epoch_tag(uint32_t epoch) { return ((epoch + 1u) >> 1) & 1u; }
__device__ __forceinline__ uint32_t tagged(float v, uint32_t tag) { return (__float_as_uint(v) & ~1u) | tag; }
__device__ __forceinline__ void publish(u32x4* slot, float a0, float s0, float a1, float s1, uint32_t epoch) {
  const uint32_t tg = epoch_tag(epoch);
  uint64_t* q = (uint64_t*)slot;
  __hip_atomic_store(q, ((uint64_t)tagged(s0, tg) << 32) | tagged(a0, tg), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(q + 1, ((uint64_t)tagged(s1, tg) << 32) | tagged(a1, tg), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ u32x4 peek(const u32x4* slot) {
  uint64_t* q = (uint64_t*)slot;
  const uint64_t lo = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t hi = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return u32x4{(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32)};
}
__device__ __forceinline__ bool fresh(const u32x4& w, uint32_t epoch) {
  const uint32_t tg = epoch_tag(epoch);
  return ((w[0] & 1u) == tg) & ((w[1] & 1u) == tg) & ((w[2] & 1u) == tg) & ((w[3] & 1u) == tg);
}

// Statistics of a workgroup's slice for one tensor, from the per-wave values
// in LDS: a = max * log2(e) (0 when the slice holds only -inf), and the sum
// of 2^{x log2e - a}.  Three data waves per workgroup; the exchange wave
// computes them for publishing and for its own use with this same code, so
// both hold identical bits.
struct SliceStats {
  float a, s;
};
__device__ __forceinline__ SliceStats slice_stats(const float* wmax, const float* wsum) {
  const float m = vmax(vmax(wmax[0], wmax[1]), wmax[2]);
  return {m == -INFINITY ? 0.f : m * kLog2e, (wsum[0] + wsum[1]) + wsum[2]};
}

// Single 32-bit exchange words (one float with its tag), in slots that rotate
// over `copies` (a power of two) epochs: a slot awaited for epoch e holds
// epoch e, epoch e - copies or the zeros of the launch, and the tag
// ((e / copies) + 1) & 1 tells e from both.
__device__ __forceinline__ uint32_t epoch_tag_n(uint32_t epoch, uint32_t copies) {
  return ((epoch / copies) + 1u) & 1u;
}
__device__ __forceinline__ void publish32(uint32_t* slot, uint32_t word) {
  __hip_atomic_store(slot, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t peek32(const uint32_t* slot) {
  return __hip_atomic_load((uint32_t*)slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---- host side
constexpr int kLdsBytesPerCU = 160 * 1024;

// Co-resident workgroups of a cluster `kernel` launched with `threads`
// threads per workgroup on the current device, cached per (device, kernel):
// the occupancy query is far slower than a launch.  The runtime's figure is
// capped by what the kernel's registers and LDS allow (four SIMDs of at most
// eight waves and 512 VGPRs per lane, allocated in blocks of 8; a
// workgroup's waves take any free slots), so a cluster never waits on a
// member that the hardware could not place.  -1 on a failed query.
inline int cluster_capacity(const void* kernel, int threads, const char* who) {
  static KeyedCache<int> cache;
  int dev = 0, have = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (cache.find(dev, kernel, have)) return have;
  int cus = 0, per = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, threads, 0) != hipSuccess) return -1;
  hipFuncAttributes attr{};
  if (hipFuncGetAttributes(&attr, kernel) != hipSuccess) return -1;
  const int waves = (threads + kWave - 1) / kWave;
  const int vgprs = ((attr.numRegs > 0 ? attr.numRegs : 1) + 7) / 8 * 8;
  const int by_regs = 4 * std::min(8, 512 / vgprs) / waves;
  const int by_lds = attr.sharedSizeBytes > 0 ? kLdsBytesPerCU / (int)attr.sharedSizeBytes : 8;
  per = std::min(per, std::min(by_regs, by_lds));
  if (getenv("DSPARK_VERBOSE"))
    fprintf(stderr, "[dspark] %s: %d VGPRs, %zu B LDS -> %d workgroups per CU\n", who, attr.numRegs,
            (size_t)attr.sharedSizeBytes, per);
  cache.put(dev, kernel, cus * per);
  return cus * per;
}

}  // namespace cluster

// Poll limit of the bounded waits inside cooperative grids (dspark_set_wait_limit).
uint32_t wait_limit();

}  // namespace dspark
