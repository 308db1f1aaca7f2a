// Markov-head sampler, all gamma steps in one persistent launch (page 1,
// "03 · DSpark 建模", §3.7, the paper's Eq. 5; page 2, "从 DFlash 到 dLLM
// Self-Spec（三）", §3.4 and §3.8.2).  Same arithmetic and results as the
// per-step kernels of markov.hip: l = base[:, i, :] + W1[prev] @ W2, greedy
// argmax or argmax l / T + Gumbel, lowest index on ties, prev <- token.
//
// Why one launch: W2 ([r, V] bf16, 77.8 MB at r = 256, V = 151936) is the
// same at every step, and the register files of the chip's compute units
// hold all of it.  A per-step launch streams W2 and the step's base slice
// (half and half of the bytes); here W2 is read from memory once, into
// registers, and a step streams only its base slice.
//
// Layout of the work: one workgroup of 8 waves per compute unit (cooperative
// launch: the grid is co-resident).  The vocabulary is cut into 16-column
// units; workgroup w owns a contiguous run of ~NU/G units, and each wave a
// contiguous run of at most five of them (38 units = 608 columns per
// workgroup at V = 151936 on 256 compute units).  A wave keeps the MFMA A
// operands of its units for every rank step in registers (5 units x 8 rank
// steps x 4 VGPRs = 160 VGPRs): out^T = W2^T E^T with
// v_mfma_f32_16x16x32_bf16, lane (n, g) owning row n of a 16-row block and
// columns 16u + 4g .. +3 of unit u, exactly as in the per-step kernel.
//
// A step, for every 16-row block of the R <= 128 rows:
//   * the block's base logits (all of the workgroup's columns) and its rows
//     of E = W1[prev] arrive in LDS by direct-to-LDS copies that every wave
//     issues a share of: three-slot rings, so two blocks are in flight while
//     one is computed (E rows XOR-swizzled by 16-byte chunk, base rows padded
//     by one piece: both read conflict-free); the first two blocks of the
//     next step's base logits are fetched during the step handshake (they do
//     not depend on the tokens);
//   * each wave runs its MFMA chains over the rank for its units, then the
//     base add, optional step-logit store, Philox Gumbel perturbation and a
//     running argmax per row, folded over the four lanes of a row and into an
//     LDS key per row.
// Step end: one device-scope atomic max per row and workgroup into the
// replicated key slots of markov_step.h (the returned values are waited for,
// so the atomics are complete), then an arrival count per step and a
// bounded wait until every workgroup has arrived; the tokens are decoded
// from the key slots with device-scope loads.  A wait that runs out sets
// DSPARK_STATUS_WAIT_TIMEOUT and goes on (not expected: the grid is
// co-resident).  The arrival counter of step i lives in the last key of
// replica 0 of step i's slots (unused: R <= 128 rows of 512 per replica).
#include <atomic>

#include "common.h"
#include "host_cache.h"
#include "markov_step.h"
#include "philox.h"

using namespace dspark;

namespace {

constexpr int kRW = 8;           // waves per workgroup
constexpr int kRT = 64 * kRW;    // threads
constexpr int kKU = 5;           // at most this many 16-column units per wave
constexpr int kKS = 8;           // at most this many 32-wide rank steps (r <= 256)
constexpr int kMaxRows = 128;
constexpr int kMaxUnitsWG = kRW * kKU;                  // 16-column units per workgroup
constexpr int kNS = 3;                                  // ring slots (two blocks in flight)
constexpr int kBSlot = 16 * (4 * kMaxUnitsWG + 1) * 16; // base logits of one 16-row block (+1 piece per row)
constexpr int kESlot = 16 * 512;                        // E rows of one block
constexpr int kLdsBytes = kNS * kBSlot + kNS * kESlot + kMaxRows * 8 + kMaxRows * 4;
static_assert(kLdsBytes <= 160 * 1024, "LDS budget");

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  const uint32_t lo = __shfl_xor((uint32_t)v, m, kWave);
  const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m, kWave);
  return ((uint64_t)hi << 32) | lo;
}

// Wait until at most n of this wave's vector memory operations are in
// flight (n wave-uniform; larger n wait as for 15, which is stricter).
__device__ __forceinline__ void wait_vmcnt_upto(int n) {
  switch (n <= 0 ? 0 : (n > 15 ? 15 : n)) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<1>(); break;
    case 2: wait_vmcnt<2>(); break;
    case 3: wait_vmcnt<3>(); break;
    case 4: wait_vmcnt<4>(); break;
    case 5: wait_vmcnt<5>(); break;
    case 6: wait_vmcnt<6>(); break;
    case 7: wait_vmcnt<7>(); break;
    case 8: wait_vmcnt<8>(); break;
    case 9: wait_vmcnt<9>(); break;
    case 10: wait_vmcnt<10>(); break;
    case 11: wait_vmcnt<11>(); break;
    case 12: wait_vmcnt<12>(); break;
    case 13: wait_vmcnt<13>(); break;
    case 14: wait_vmcnt<14>(); break;
    default: wait_vmcnt<15>(); break;
  }
}

// LDS accesses of the step loop are written as inline assembly.  The
// compiler orders every LDS read after ALL direct-to-LDS copies in flight
// (vmcnt(0): it cannot tell the copies' targets apart), which would drain
// the rings before every operand read; here the copies are waited for
// explicitly, per block.  Each read statement also waits for its own
// results (lgkmcnt(0)) so that no register is touched while in flight.
__device__ __forceinline__ uint32_t lds_off(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ void lds_read2(uint32_t a0, uint32_t a1, u32x4& x0, u32x4& x1) {
  asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %3\n\ts_waitcnt lgkmcnt(0)"
               : "=&v"(x0), "=&v"(x1) : "v"(a0), "v"(a1) : "memory");
}
__device__ __forceinline__ void lds_read4(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3, u32x4& x0,
                                          u32x4& x1, u32x4& x2, u32x4& x3) {
  asm volatile(
      "ds_read_b128 %0, %4\n\tds_read_b128 %1, %5\n\tds_read_b128 %2, %6\n\tds_read_b128 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(x0), "=&v"(x1), "=&v"(x2), "=&v"(x3)
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3)
      : "memory");
}
__device__ __forceinline__ void lds_read5(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3, uint32_t a4,
                                          u32x4& x0, u32x4& x1, u32x4& x2, u32x4& x3, u32x4& x4) {
  asm volatile(
      "ds_read_b128 %0, %5\n\tds_read_b128 %1, %6\n\tds_read_b128 %2, %7\n\tds_read_b128 %3, %8\n\t"
      "ds_read_b128 %4, %9\n\ts_waitcnt lgkmcnt(0)"
      : "=&v"(x0), "=&v"(x1), "=&v"(x2), "=&v"(x3), "=&v"(x4)
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3), "v"(a4)
      : "memory");
}
__device__ __forceinline__ int lds_read_i32(uint32_t a0) {
  int x;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(x) : "v"(a0) : "memory");
  return x;
}
__device__ __forceinline__ uint64_t lds_read_u64(uint32_t a0) {
  uint64_t x;
  asm volatile("ds_read_b64 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(x) : "v"(a0) : "memory");
  return x;
}
__device__ __forceinline__ void lds_write_u64(uint32_t a0, uint64_t x) {
  asm volatile("ds_write_b64 %0, %1\n\ts_waitcnt lgkmcnt(0)" :: "v"(a0), "v"(x) : "memory");
}
__device__ __forceinline__ void lds_write_i32(uint32_t a0, int x) {
  asm volatile("ds_write_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" :: "v"(a0), "v"(x) : "memory");
}
// LDS atomic max without a wait (LDS operations complete in order; the step
// end waits for them before the keys are read)
__device__ __forceinline__ void lds_max_u64_nowait(uint32_t a0, uint64_t x) {
  asm volatile("ds_max_u64 %0, %1" :: "v"(a0), "v"(x) : "memory");
}
__device__ __forceinline__ void lds_wait_all() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

struct RoundArgs {
  const float* base;
  const uint16_t* w1;
  const uint16_t* w2;
  const int32_t* first_prev;
  int32_t* tokens;
  float* step_logits;
  uint64_t* keys;
  int32_t* status;
  int R, gamma, V, r;
  float invT;
  uint32_t seed_lo, seed_hi;
  uint32_t spin_limit;
};

template <bool kGumbel>
__global__ __launch_bounds__(kRT) __attribute__((amdgpu_waves_per_eu(2, 2))) void markov_round_mfma(RoundArgs a) {
  __shared__ __align__(16) unsigned char bring[kNS * kBSlot];  // base logits, three 16-row blocks
  __shared__ __align__(16) unsigned char ering[kNS * kESlot];  // E rows, three 16-row blocks
  __shared__ uint64_t rowkey[kMaxRows];
  __shared__ int32_t prevtok[kMaxRows];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int R = a.R, gamma = a.gamma, V = a.V, r = a.r;
  const int nrb = (R + 15) / 16;
  const int ks = r / 32;  // rank steps (r % 32 == 0, checked on the host)
  const int G = (int)gridDim.x;

  // ---- this workgroup's units [U0, U1) and this wave's [ua, ua + nu)
  const int NU = (V + 15) / 16;
  const int U0 = (int)((int64_t)blockIdx.x * NU / G), U1 = (int)((int64_t)(blockIdx.x + 1) * NU / G);
  const int nuw = U1 - U0;  // <= kMaxUnitsWG, checked on the host
  const int ua = __builtin_amdgcn_readfirstlane(U0 + wave * nuw / kRW);
  const int nu = __builtin_amdgcn_readfirstlane(U0 + (wave + 1) * nuw / kRW - ua);  // 0 .. kKU
  const int pitch = 4 * nuw + 1;                   // base ring row pitch in 16-byte pieces
  const int npieces = nuw > 0 ? 16 * pitch : 0;    // pieces per base block (the last of each row is padding)
  const int ninst = (npieces + 63) / 64;           // 1 KB copies per base block
  const int my_inst = (ninst - wave + kRW - 1) / kRW;  // this wave's share: copies wave, wave + 8, ...

  // ---- copies.  `issued` counts this wave's direct-to-LDS copies; a copy group is waited for with
  //      vmcnt(issued - count after the group) (vector memory operations complete in order)
  uint32_t issued = 0;

  // ---- W2 operands: A[u][kk], lane (n, g) holds W2[32kk + 8g + e][16(ua + u) + n], e = 0..7,
  //      built through LDS one rank step at a time: the 32 rank rows of the workgroup's columns
  //      come in by direct-to-LDS copies (two rank steps in flight, in the base ring's space;
  //      rows padded by one 16-byte piece), and the transposing read gives the operand layout.
  //      Units past nu and rank steps past r are zero; columns past V hold copies of column
  //      V - 8 .. V - 1, whose products are never used.
  u32x4 A[kKU][kKS];
  {
    const int spc = 2 * nuw + 1;          // 16-byte pieces per staged rank row (last: padding)
    const int spitch = spc * 16;
    const int nwi = (32 * spc + 63) / 64;  // 1 KB copies per rank step
    const int my_w = nuw > 0 ? (nwi - wave + kRW - 1) / kRW : 0;
    auto stage = [&](int kk) -> unsigned char* { return bring + (kk & 1) * (kNS * kBSlot / 2); };
    auto issue_w2 = [&](int kk) {
      unsigned char* dst = stage(kk);
      for (int jj = 0; jj < my_w; ++jj) {
        const int i = wave + jj * kRW;
        const int p = i * 64 + lane;
        if (p < 32 * spc) {
          const int row = p / spc;
          int q = p - row * spc;
          q = q < 2 * nuw ? q : 2 * nuw - 1;
          const int col = min(U0 * 16 + q * 8, V - 8);
          __builtin_amdgcn_global_load_lds((const void*)(a.w2 + (int64_t)(32 * kk + row) * V + col),
                                           (lds_void*)(dst + i * 1024), 16, 0, 0);
        }
      }
      issued += my_w;
    };
    uint32_t done_at[2] = {0, 0};
    issue_w2(0);
    done_at[0] = issued;
    if (ks > 1) {
      issue_w2(1);
      done_at[1] = issued;
    }
    const int ul = ua - U0;
#pragma unroll
    for (int kk = 0; kk < kKS; ++kk) {
      if (kk < ks) {
        wait_vmcnt_upto((int)(issued - done_at[kk & 1]));
        block_barrier();  // every wave's copies of rank step kk have landed
        const unsigned char* stg = stage(kk);
#pragma unroll
        for (int u = 0; u < kKU; ++u) {
          u32x4 v = u32x4{0u, 0u, 0u, 0u};
          if (u < nu) {
            const unsigned char* ap = stg + (8 * g + n / 4) * spitch + 8 * (n % 4) + 32 * (ul + u);
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)ap);
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(ap + 4 * spitch));
            const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
            v = u32x4{l2.x, l2.y, h2.x, h2.y};
          }
          A[u][kk] = v;
        }
        __syncthreads();  // every wave is done with this stage buffer
        if (kk + 2 < ks) {
          issue_w2(kk + 2);
          done_at[kk & 1] = issued;
        }
      } else {
#pragma unroll
        for (int u = 0; u < kKU; ++u) A[u][kk] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }

  // last_b / last_e: the copy count after each ring slot's latest copies
  uint32_t last_b[kNS] = {0, 0, 0}, last_e[kNS] = {0, 0, 0};
  // base block rb of step st into slot: piece p = q * pitch + c (row q of the block, column piece c;
  // c == 4 nuw is padding, filled with a duplicate of the row's last piece)
  // (q = p / pitch through a float reciprocal: exact here, since p < 2^12 and (p + 1/2) / pitch
  // stays at least 1 / (2 pitch) away from an integer)
  const float inv_pitch = 1.0f / (float)pitch;
  const int64_t gV = (int64_t)gamma * V;
  auto issue_base = [&](int st, int rb, int slot) {
    unsigned char* dst = bring + slot * kBSlot;
    const float* src0 = a.base + (int64_t)st * V;
    for (int j = 0; j < my_inst; ++j) {
      const int i = wave + j * kRW;
      int p = i * 64 + lane;
      asm volatile("" : "+v"(p));  // recomputed per copy: keeps these lane offsets out of the loop's registers
      if (p < npieces) {
        const int q = (int)(((float)p + 0.5f) * inv_pitch);
        int c = p - q * pitch;
        c = c < 4 * nuw ? c : 4 * nuw - 1;
        const int row = min(rb * 16 + q, R - 1);
        const int col = min(U0 * 16 + 4 * c, V - 4);
        __builtin_amdgcn_global_load_lds((const void*)(src0 + (int64_t)row * gV + col),
                                         (lds_void*)(dst + i * 1024), 16, 0, 0);
      }
    }
    issued += my_inst;
    last_b[slot] = issued;
  };
  // E rows of block rb into slot: copy `wave` covers block rows 2 wave and 2 wave + 1; lane l
  // stores chunk (l & 31) of its row, which holds the row's W1 chunk (l & 31) ^ (row & 15)
  const int ksc = r / 8;  // 16-byte chunks per W1 row
  const uint32_t tok_lds = lds_off(prevtok);
  auto issue_e = [&](int rb, int slot) {
    const int q = 2 * wave + (lane >> 5);
    const int tok = lds_read_i32(tok_lds + 4 * min(rb * 16 + q, kMaxRows - 1));
    int c = (lane & 31) ^ q;
    c = c < ksc ? c : c % ksc;  // chunks beyond the rank are never read
    __builtin_amdgcn_global_load_lds((const void*)(a.w1 + (int64_t)tok * r + c * 8),
                                     (lds_void*)(ering + slot * kESlot + wave * 1024), 16, 0, 0);
    issued += 1;
    last_e[slot] = issued;
  };

  // ---- prologue: the anchors' tokens, zero row keys, the first two base blocks in flight
  if (threadIdx.x < kMaxRows) {
    const int t = threadIdx.x;
    int p = 0;
    if (t < R) {
      p = a.first_prev[t];
      if (p < 0 || p >= V) {
        if (blockIdx.x == 0) status_or(a.status, DSPARK_STATUS_BAD_TOKEN);
        p = 0;
      }
    }
    prevtok[t] = p;
    rowkey[t] = 0ull;
  }
  __syncthreads();
  issue_base(0, 0, 0);
  if (nrb > 1) issue_base(0, 1, 1);

  const uint32_t key_lds = lds_off(rowkey);
  const uint32_t bring_lds = lds_off(bring), ering_lds = lds_off(ering);
  for (int st = 0; st < gamma; ++st) {
    // E rows of the step's first two blocks (the tokens are known now)
    issue_e(0, 0);
    if (nrb > 1) issue_e(1, 1);

    for (int rb = 0; rb < nrb; ++rb) {
      const int j = st * nrb + rb;  // block index over the whole launch: base slot j % 3
      const int bs = j % kNS, es = rb % kNS;
      {
        const uint32_t need = last_b[bs] > last_e[es] ? last_b[bs] : last_e[es];
        wait_vmcnt_upto((int)(issued - need));
      }
      // every wave's copies of this block have landed, and every wave is done with block rb - 1,
      // whose slots take block rb + 2
      block_barrier();
      if (rb + 2 < nrb) {
        issue_base(st, rb + 2, (j + 2) % kNS);
        issue_e(rb + 2, (rb + 2) % kNS);
      }
      if (nu > 0) {
        const int row = rb * 16 + n;
        const uint32_t erow = ering_lds + es * kESlot + n * 512, swz = (uint32_t)n;
        f32x4 acc[kKU];
#pragma unroll
        for (int u = 0; u < kKU; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < kKS; kk += 4) {
          if (kk < ks) {  // ks is a multiple of 1 .. 8 rank steps; missing ones read zeros' partners
            u32x4 e0, e1, e2, e3;
            lds_read4(erow + (((4 * kk + g) ^ swz) << 4), erow + (((4 * kk + 4 + g) ^ swz) << 4),
                      erow + (((4 * kk + 8 + g) ^ swz) << 4), erow + (((4 * kk + 12 + g) ^ swz) << 4), e0, e1, e2,
                      e3);
#pragma unroll
            for (int u = 0; u < kKU; ++u) acc[u] = mfma16x16x32(A[u][kk], e0, acc[u]);
#pragma unroll
            for (int u = 0; u < kKU; ++u) acc[u] = mfma16x16x32(A[u][kk + 1], e1, acc[u]);
#pragma unroll
            for (int u = 0; u < kKU; ++u) acc[u] = mfma16x16x32(A[u][kk + 2], e2, acc[u]);
#pragma unroll
            for (int u = 0; u < kKU; ++u) acc[u] = mfma16x16x32(A[u][kk + 3], e3, acc[u]);
          }
        }
        // the lane's base logits of its units (a unit past nu re-reads unit 0: unused)
        const uint32_t sl = bring_lds + bs * kBSlot + (n * pitch + 4 * (ua - U0) + g) * 16;
        u32x4 bw[kKU];
        lds_read5(sl, sl + (nu > 1 ? 64 : 0), sl + (nu > 2 ? 128 : 0), sl + (nu > 3 ? 192 : 0),
                  sl + (nu > 4 ? 256 : 0), bw[0], bw[1], bw[2], bw[3], bw[4]);
        float bz = -INFINITY;
        uint32_t bv = 0xffffffffu;
#pragma unroll
        for (int u = 0; u < kKU; ++u) {
          if (u < nu) {
            const f32x4 b = __builtin_bit_cast(f32x4, bw[u]);
            const int c0 = (ua + u) * 16 + 4 * g;
            const f32x4 l = acc[u] + b;
            const bool ok = row < R && c0 < V;
            if (a.step_logits && ok) *(f32x4*)(a.step_logits + ((int64_t)row * gamma + st) * V + c0) = l;
            f32x4 z = l;
            if constexpr (kGumbel) {
              const u32x4 x = philox4x32_10(u32x4{(uint32_t)(c0 >> 2), (uint32_t)st, (uint32_t)row, 0u},
                                            a.seed_lo, a.seed_hi);
#pragma unroll
              for (int e = 0; e < 4; ++e) z[e] = fmaf(l[e], a.invT, gumbel_from_bits(x[e]));
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const bool better = ok && z[e] > bz;
              bz = better ? z[e] : bz;
              bv = better ? (uint32_t)(c0 + e) : bv;
            }
          }
        }
        // each lane folds its own key into the row's LDS key (the four lanes of a row meet there)
        if (bv != 0xffffffffu) lds_max_u64_nowait(key_lds + 8 * row, argmax_key(bz, bv));
      }
    }
    lds_wait_all();
    __syncthreads();

    // ---- step end: fold into the device key slots, arrive, prefetch, wait, decode
    uint64_t* ks_st = a.keys + (int64_t)st * keys_per_step(R);
    if (threadIdx.x < R) {
      const uint64_t key = rowkey[threadIdx.x];
      rowkey[threadIdx.x] = 0ull;
      if (key) {
        uint64_t* dst = ks_st + (int64_t)(blockIdx.x % kKeyReplicas) * replica_stride(R) + threadIdx.x;
        const uint64_t seen = __hip_atomic_fetch_max(dst, key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (seen == ~0ull) status_or(a.status, 0);  // the returned value is waited for: the atomic is complete
      }
    }
    __syncthreads();
    uint32_t* arrive = (uint32_t*)(ks_st + replica_stride(R) - 1);
    if (threadIdx.x == 0) __hip_atomic_fetch_add(arrive, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (st + 1 < gamma) {  // the next step's first two base blocks (their slots are free: all waves passed)
      issue_base(st + 1, 0, ((st + 1) * nrb) % kNS);
      if (nrb > 1) issue_base(st + 1, 1, ((st + 1) * nrb + 1) % kNS);
    }
    if (threadIdx.x == 0) {
      uint32_t spins = 0;
      while (__hip_atomic_load(arrive, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < (uint32_t)G) {
        if (++spins > a.spin_limit) {
          status_or(a.status, DSPARK_STATUS_WAIT_TIMEOUT);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    block_barrier();
    if (threadIdx.x < R) {
      const int t = threadIdx.x;
      uint64_t x[kKeyReplicas];  // all replicas in flight together, then folded
#pragma unroll
      for (int q = 0; q < kKeyReplicas; ++q)
        x[q] = __hip_atomic_load(ks_st + q * replica_stride(R) + t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      uint64_t k = 0;
#pragma unroll
      for (int q = 0; q < kKeyReplicas; ++q) k = x[q] > k ? x[q] : k;
      uint32_t tok = k ? argmax_key_index(k) : 0xffffffffu;
      if (tok >= (uint32_t)V) {
        if (blockIdx.x == 0) status_or(a.status, DSPARK_STATUS_BAD_TOKEN);
        tok = 0;
      }
      lds_write_i32(tok_lds + 4 * t, (int)tok);
      if (blockIdx.x == 0) a.tokens[(int64_t)t * gamma + st] = (int32_t)tok;
    }
    block_barrier();
  }
}

struct Capacity {
  int cus = 0, per_cu = 0;
};

// Compute units and co-resident workgroups of the round kernel per device
// (cached: the queries cost far more than a launch).
Capacity round_capacity(const void* kern) {
  static KeyedCache<Capacity> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return {};
  Capacity c;
  if (cache.find(dev, kern, c)) return c;
  if (hipDeviceGetAttribute(&c.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return {};
  int coop = 0;
  if (hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess || !coop) c.cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&c.per_cu, kern, kRT, 0) != hipSuccess) c.per_cu = 0;
  cache.put(dev, kern, c);
  return c;
}


// ---------------------------------------------------------------------------
// Teacher-forced logits of N independent rows (page 2, "从 DFlash 到 dLLM
// Self-Spec（三）", §3.4: every position of a training block takes the true
// previous token): one Markov step per row, prev from the caller, logits
// stored (optionally soft-capped, c tanh(l / c)) and each row's greedy argmax
// folded into the key slots.  Same layout of the work as the round kernel:
// W2 in registers (read once per launch), every workgroup streams all row
// blocks of its vocabulary columns, base logits and E rows through three-slot
// rings of direct-to-LDS copies.  There is no dependency between row blocks,
// so no wait on other workgroups: an ordinary launch.  The E rows' tokens are
// read with scalar loads (two per wave and block), whose waits do not hold
// the copies in flight.
struct RowsArgs {
  const float* base;
  const uint16_t* w1;
  const uint16_t* w2;
  const int32_t* prev;
  float* logits;
  uint64_t* keys;
  int32_t* status;
  int N, V, r;
  float invc;  // 1 / softcap
};

template <bool kSoftcap>
__global__ __launch_bounds__(kRT) __attribute__((amdgpu_waves_per_eu(2, 2))) void markov_rows_mfma(RowsArgs a) {
  __shared__ __align__(16) unsigned char bring[kNS * kBSlot];  // base logits, three 16-row blocks
  __shared__ __align__(16) unsigned char ering[kNS * kESlot];  // E rows, three 16-row blocks
  __shared__ __align__(16) uint64_t rowkey[2 * 16];           // row keys of the last two blocks

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int N = a.N, V = a.V, r = a.r;
  const int nrb = (N + 15) / 16;
  const int ks = r / 32;
  const int G = (int)gridDim.x;

  const int NU = (V + 15) / 16;
  const int U0 = (int)((int64_t)blockIdx.x * NU / G), U1 = (int)((int64_t)(blockIdx.x + 1) * NU / G);
  const int nuw = U1 - U0;
  const int ua = __builtin_amdgcn_readfirstlane(U0 + wave * nuw / kRW);
  const int nu = __builtin_amdgcn_readfirstlane(U0 + (wave + 1) * nuw / kRW - ua);
  const int pitch = 4 * nuw + 1;
  const int npieces = nuw > 0 ? 16 * pitch : 0;
  const int ninst = (npieces + 63) / 64;
  const int my_inst = (ninst - wave + kRW - 1) / kRW;
  uint32_t issued = 0;

  // ---- W2 operands in registers, as in the round kernel
  u32x4 A[kKU][kKS];
  {
    const int spc = 2 * nuw + 1;
    const int spitch = spc * 16;
    const int nwi = (32 * spc + 63) / 64;
    const int my_w = nuw > 0 ? (nwi - wave + kRW - 1) / kRW : 0;
    auto stage = [&](int kk) -> unsigned char* { return bring + (kk & 1) * (kNS * kBSlot / 2); };
    auto issue_w2 = [&](int kk) {
      unsigned char* dst = stage(kk);
      for (int jj = 0; jj < my_w; ++jj) {
        const int i = wave + jj * kRW;
        const int p = i * 64 + lane;
        if (p < 32 * spc) {
          const int row = p / spc;
          int q = p - row * spc;
          q = q < 2 * nuw ? q : 2 * nuw - 1;
          const int col = min(U0 * 16 + q * 8, V - 8);
          __builtin_amdgcn_global_load_lds((const void*)(a.w2 + (int64_t)(32 * kk + row) * V + col),
                                           (lds_void*)(dst + i * 1024), 16, 0, 0);
        }
      }
      issued += my_w;
    };
    uint32_t done_at[2] = {0, 0};
    issue_w2(0);
    done_at[0] = issued;
    if (ks > 1) {
      issue_w2(1);
      done_at[1] = issued;
    }
    const int ul = ua - U0;
#pragma unroll
    for (int kk = 0; kk < kKS; ++kk) {
      if (kk < ks) {
        wait_vmcnt_upto((int)(issued - done_at[kk & 1]));
        block_barrier();
        const unsigned char* stg = stage(kk);
#pragma unroll
        for (int u = 0; u < kKU; ++u) {
          u32x4 v = u32x4{0u, 0u, 0u, 0u};
          if (u < nu) {
            const unsigned char* ap = stg + (8 * g + n / 4) * spitch + 8 * (n % 4) + 32 * (ul + u);
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)ap);
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(ap + 4 * spitch));
            const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
            v = u32x4{l2.x, l2.y, h2.x, h2.y};
          }
          A[u][kk] = v;
        }
        __syncthreads();
        if (kk + 2 < ks) {
          issue_w2(kk + 2);
          done_at[kk & 1] = issued;
        }
      } else {
#pragma unroll
        for (int u = 0; u < kKU; ++u) A[u][kk] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }

  uint32_t last_b[kNS] = {0, 0, 0}, last_e[kNS] = {0, 0, 0};
  const float inv_pitch = 1.0f / (float)pitch;
  auto issue_base = [&](int rb, int slot) {
    unsigned char* dst = bring + slot * kBSlot;
    for (int j = 0; j < my_inst; ++j) {
      const int i = wave + j * kRW;
      int p = i * 64 + lane;
      asm volatile("" : "+v"(p));
      if (p < npieces) {
        const int q = (int)(((float)p + 0.5f) * inv_pitch);
        int c = p - q * pitch;
        c = c < 4 * nuw ? c : 4 * nuw - 1;
        const int row = min(rb * 16 + q, N - 1);
        const int col = min(U0 * 16 + 4 * c, V - 4);
        __builtin_amdgcn_global_load_lds((const void*)(a.base + (int64_t)row * V + col),
                                         (lds_void*)(dst + i * 1024), 16, 0, 0);
      }
    }
    issued += my_inst;
    last_b[slot] = issued;
  };
  // E rows of block rb: copy `wave` covers block rows 2 wave and 2 wave + 1, whose tokens come in by
  // scalar loads; lane l stores chunk l & 31 of its row, which holds W1 chunk (l & 31) ^ (row & 15)
  typedef const __attribute__((address_space(4))) int32_t const_i32;
  const const_i32* prev_c = (const const_i32*)a.prev;
  const int ksc = r / 8;
  auto issue_e = [&](int rb, int slot) {
    const int r0 = min(rb * 16 + 2 * wave, N - 1), r1 = min(rb * 16 + 2 * wave + 1, N - 1);
    int t0 = prev_c[r0], t1 = prev_c[r1];
    if ((uint32_t)t0 >= (uint32_t)V || (uint32_t)t1 >= (uint32_t)V) {
      if (blockIdx.x == 0 && lane == 0) status_or(a.status, DSPARK_STATUS_BAD_TOKEN);
      t0 = (uint32_t)t0 < (uint32_t)V ? t0 : 0;
      t1 = (uint32_t)t1 < (uint32_t)V ? t1 : 0;
    }
    const int q = 2 * wave + (lane >> 5);
    const int tok = (lane >> 5) ? t1 : t0;
    int c = (lane & 31) ^ q;
    c = c < ksc ? c : c % ksc;
    __builtin_amdgcn_global_load_lds((const void*)(a.w1 + (int64_t)tok * r + c * 8),
                                     (lds_void*)(ering + slot * kESlot + wave * 1024), 16, 0, 0);
    issued += 1;
    last_e[slot] = issued;
  };

  if (threadIdx.x < 32) rowkey[threadIdx.x] = 0ull;
  __syncthreads();
  issue_base(0, 0);
  issue_e(0, 0);
  if (nrb > 1) {
    issue_base(1, 1);
    issue_e(1, 1);
  }

  const uint32_t key_lds = lds_off(rowkey);
  const uint32_t bring_lds = lds_off(bring), ering_lds = lds_off(ering);
  const int64_t rstr = replica_stride(N);
  // the keys of block rb (final after the barrier that follows its products) -> device slots
  auto flush = [&](int rb) {
    if (wave == 0 && lane < 16) {
      const uint32_t kr = key_lds + 8 * ((rb & 1) * 16 + lane);
      const uint64_t key = lds_read_u64(kr);
      lds_write_u64(kr, 0ull);
      const int row = rb * 16 + lane;
      if (row < N && key)
        __hip_atomic_fetch_max(a.keys + (int64_t)(blockIdx.x % kKeyReplicas) * rstr + row, key, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
  };
  for (int rb = 0; rb < nrb; ++rb) {
    const int sl = rb % kNS;
    {
      const uint32_t need = last_b[sl] > last_e[sl] ? last_b[sl] : last_e[sl];
      wait_vmcnt_upto((int)(issued - need));
    }
    lds_wait_all();  // this wave's key folds of block rb - 1 have completed
    block_barrier();
    if (rb > 0) flush(rb - 1);
    if (rb + 2 < nrb) {
      issue_base(rb + 2, (rb + 2) % kNS);
      issue_e(rb + 2, (rb + 2) % kNS);
    }
    if (nu > 0) {
      const int row = rb * 16 + n;
      const uint32_t erow = ering_lds + sl * kESlot + n * 512, swz = (uint32_t)n;
      f32x4 acc[kKU];
#pragma unroll
      for (int u = 0; u < kKU; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < kKS; kk += 4) {
        if (kk < ks) {
          u32x4 e0, e1, e2, e3;
          lds_read4(erow + (((4 * kk + g) ^ swz) << 4), erow + (((4 * kk + 4 + g) ^ swz) << 4),
                    erow + (((4 * kk + 8 + g) ^ swz) << 4), erow + (((4 * kk + 12 + g) ^ swz) << 4), e0, e1, e2,
                    e3);
#pragma unroll
          for (int u = 0; u < kKU; ++u) acc[u] = mfma16x16x32(A[u][kk], e0, acc[u]);
#pragma unroll
          for (int u = 0; u < kKU; ++u) acc[u] = mfma16x16x32(A[u][kk + 1], e1, acc[u]);
#pragma unroll
          for (int u = 0; u < kKU; ++u) acc[u] = mfma16x16x32(A[u][kk + 2], e2, acc[u]);
#pragma unroll
          for (int u = 0; u < kKU; ++u) acc[u] = mfma16x16x32(A[u][kk + 3], e3, acc[u]);
        }
      }
      const uint32_t slb = bring_lds + sl * kBSlot + (n * pitch + 4 * (ua - U0) + g) * 16;
      u32x4 bw[kKU];
      lds_read5(slb, slb + (nu > 1 ? 64 : 0), slb + (nu > 2 ? 128 : 0), slb + (nu > 3 ? 192 : 0),
                slb + (nu > 4 ? 256 : 0), bw[0], bw[1], bw[2], bw[3], bw[4]);
      float bz = -INFINITY;
      uint32_t bv = 0xffffffffu;
#pragma unroll
      for (int u = 0; u < kKU; ++u) {
        if (u < nu) {
          const int c0 = (ua + u) * 16 + 4 * g;
          f32x4 l = acc[u] + __builtin_bit_cast(f32x4, bw[u]);
          if constexpr (kSoftcap) {
#pragma unroll
            for (int e = 0; e < 4; ++e) l[e] = tanhf(l[e] * a.invc) / a.invc;
          }
          const bool ok = row < N && c0 < V;
          if (ok) *(f32x4*)(a.logits + (int64_t)row * V + c0) = l;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bool better = ok && l[e] > bz;
            bz = better ? l[e] : bz;
            bv = better ? (uint32_t)(c0 + e) : bv;
          }
        }
      }
      if (bv != 0xffffffffu) lds_max_u64_nowait(key_lds + 8 * ((rb & 1) * 16 + n), argmax_key(bz, bv));
    }
  }
  lds_wait_all();
  block_barrier();
  if (nrb > 0) flush(nrb - 1);
}

}  // namespace

namespace dspark {

bool markov_round_eligible(int R, int gamma, int V, int r, const void* base, const void* w1, const void* w2,
                           const void* step_logits) {
  if (R < 1 || R > kMaxRows || gamma < 1 || r < 32 || r > 32 * kKS || r % 32 || V < 16 || V % 8) return false;
  if (((uintptr_t)base | (uintptr_t)w1 | (uintptr_t)w2 | (uintptr_t)step_logits) % 16) return false;
  return true;
}

hipError_t markov_round_launch(const float* base, const uint16_t* w1, const uint16_t* w2, const int32_t* first_prev,
                               int32_t* tokens, float* step_logits, int R, int gamma, int V, int r, float invT,
                               int greedy, uint32_t slo, uint32_t shi, uint64_t* keys, uint32_t spin_limit,
                               int32_t* status, hipStream_t s) {
  const void* kern = greedy ? (const void*)markov_round_mfma<false> : (const void*)markov_round_mfma<true>;
  const Capacity cap = round_capacity(kern);
  if (cap.cus <= 0 || cap.per_cu < 1) return hipErrorNotSupported;
  const int G = cap.cus;
  const int NU = (V + 15) / 16;
  // every workgroup owns 1 .. kMaxUnitsWG units (at most kKU per wave)
  if (NU < G || (NU + G - 1) / G > kMaxUnitsWG) return hipErrorNotSupported;
  RoundArgs args{base, w1, w2, first_prev, tokens, step_logits, keys, status, R, gamma, V, r, invT, slo, shi,
                 spin_limit};
  void* params[] = {(void*)&args};
  return hipLaunchCooperativeKernel(kern, dim3((unsigned)G), dim3(kRT), params, 0, s);
}


bool markov_rows_eligible(int N, int V, int r, const void* base, const void* w1, const void* w2, const void* logits) {
  if (N < 1 || r < 32 || r > 32 * kKS || r % 32 || V < 16 || V % 8) return false;
  if (((uintptr_t)base | (uintptr_t)w1 | (uintptr_t)w2 | (uintptr_t)logits) % 16) return false;
  return true;
}

hipError_t markov_rows_launch(const float* base, const uint16_t* w1, const uint16_t* w2, const int32_t* prev,
                              float* logits, int N, int V, int r, float softcap, uint64_t* keys, int32_t* status,
                              hipStream_t s) {
  const Capacity cap =
      round_capacity(softcap > 0.f ? (const void*)markov_rows_mfma<true> : (const void*)markov_rows_mfma<false>);
  const int cus = cap.cus;
  if (cus <= 0 || cap.per_cu < 1) return hipErrorNotSupported;
  const int NU = (V + 15) / 16;
  if (NU < cus || (NU + cus - 1) / cus > kMaxUnitsWG) return hipErrorNotSupported;
  RowsArgs args{base, w1, w2, prev, logits, keys, status, N, V, r, softcap > 0.f ? 1.f / softcap : 1.f};
  if (softcap > 0.f)
    hipLaunchKernelGGL(markov_rows_mfma<true>, dim3((unsigned)cus), dim3(kRT), 0, s, args);
  else
    hipLaunchKernelGGL(markov_rows_mfma<false>, dim3((unsigned)cus), dim3(kRT), 0, s, args);
  return hipGetLastError();
}

}  // namespace dspark
