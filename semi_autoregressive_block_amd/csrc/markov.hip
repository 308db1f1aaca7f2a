// Markov-head sequential sampler (page 1, "03 · DSpark 建模", §3.7, the
// paper's Eq. 5; page 2, "从 DFlash 到 dLLM Self-Spec（三）", §3.4 and
// §3.8.2).
//
// For gamma steps, every row takes l = base[:, i, :] + W1[prev] @ W2 over the
// whole vocabulary, picks argmax l (greedy) or argmax l/T + Gumbel, and feeds
// the token forward.  Each step is one kernel launch:
//
// * The rank-r x V product is an MFMA contraction over the rank (bf16 in,
//   fp32 accumulate, v_mfma_f32_16x16x32_bf16), computed transposed so that
//   each lane owns one row and four columns per 16-column product; W2 tiles
//   are staged in LDS and read with the transposing LDS read, E = W1[prev]
//   stays in registers.
// * 64-column tiles are handed out interleaved over the workgroups (the step
//   streams W2 and its base slice exactly once); the base add, the optional
//   step-logit store, the Philox Gumbel perturbation and the argmax are fused
//   into each tile's epilogue, with a running (value, index) best per row.
// * Row maxima are folded with 64-bit keys (order-preserving float bits,
//   then the inverted index so ties go to the lowest index): shuffles, then
//   one device-scope atomic max per row and workgroup into one of 16 replica
//   slots of the row (memory-side atomics on one address serialise; replicas
//   spread them).  The next step decodes prev from the maximum over the
//   replicas on the device; there is no host round trip inside the gamma
//   loop.
#include <atomic>

#include "common.h"
#include "host_cache.h"
#include "philox.h"
#include "markov_step.h"

using namespace dspark;

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  const uint32_t lo = __shfl_xor((uint32_t)v, m, kWave);
  const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m, kWave);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ int decode_prev(const uint64_t* keys_prev, const int32_t* first_prev,
                                           int row, int R, int V, int32_t* status) {
  int p;
  if (keys_prev) {
    p = (int)argmax_key_index(read_key(keys_prev, row, R));
  } else {
    p = first_prev[row];
  }
  if (p < 0 || p >= V) {
    status_or(status, DSPARK_STATUS_BAD_TOKEN);
    p = 0;
  }
  return p;
}

__device__ __forceinline__ void fold_key_global(uint64_t* keys, int row, int R, uint64_t key) {
  uint64_t* dst = keys + (int64_t)(blockIdx.x % kKeyReplicas) * replica_stride(R) + row;
  atomicMax((unsigned long long*)dst, (unsigned long long)key);
}

// ----------------------------------------------------------------- MFMA path
// NW waves per workgroup, 16 rows per wave (row group = 16*NW rows), KS
// 32-wide rank steps (rank padded with zeros to 32*KS).  The vocabulary is
// cut into 64-column tiles handed out interleaved: at step t of its loop
// each workgroup owns one tile of round t*grid .. t*grid + grid-1, so the
// workgroups running side by side read one contiguous span of every W2 row
// and every base row.
//
// The product is computed transposed, out^T = W2^T E^T: W2^T is the A operand
// (v_mfma_f32_16x16x32_bf16), read from the LDS copy of the tile with
// ds_read_b64_tr_b16, and E^T = W1[prev]^T is the B operand, held in
// registers.  Lane (n, g) of a wave then owns row n of the wave's 16 and,
// for product j, columns 16j + 4g .. +3 of the tile: its base logits are
// four 16-byte loads and its argmax is lane-local until the final fold.
//
// Loads: NS register sets hold tiles t .. t+NS-1 (W2 pieces and the lane's
// base logits).  Iteration t computes tile t from LDS, issues tile t + NS's
// loads into the freed set and moves tile t + 1's W2 into the other LDS
// buffer.  A compute unit accepts only a few tens of KB of outstanding loads
// and a wave stalls at a load it cannot issue, so more sets mostly delay the
// first tile; two sets are used for 128-row workgroups.  Every global load is
// unconditional from a clamped, always-valid address (invalid lanes are
// zeroed after the load).  With FL the base logits are fetched as whole
// 128-byte lines (the request count, not only the bytes, bounds a compute
// unit's streaming rate) and regathered into the MFMA layout through LDS.
// The step's dependent reads (the previous step's keys, then the W1 rows
// they select) go out right after tile 0, ahead of the other tiles.
constexpr int kTileCols = 64;
constexpr int kLdsRow = 144;  // bytes per staged W2 row of a tile (128 + 16: spreads LDS banks)

// SC: soft-capped logits c * tanh(l / c) (block logits only; sampling is then
// greedy and the temperature argument carries 1 / c).
// EB: the rank-r row of each row is read from `ebuf` ([R, gamma, r] float32,
// rounded to bf16 here) instead of gathered from W1 by the previous token
// (the gated and recurrent heads compute it beforehand).
template <int NW, int KS, int NS, bool FL, bool SC = false, bool EB = false>
__global__ __launch_bounds__(64 * NW) void markov_step_mfma(
    const float* __restrict__ base, const uint16_t* __restrict__ w1, const float* __restrict__ ebuf,
    const uint16_t* __restrict__ w2, const int32_t* __restrict__ first_prev,
    const uint64_t* __restrict__ keys_prev, uint64_t* __restrict__ keys_out,
    float* __restrict__ step_logits, int R, int gamma, int V, int r, int step, float invT,
    int greedy, uint32_t seed_lo, uint32_t seed_hi, int32_t* __restrict__ status) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int NT = 64 * NW;                // threads
  constexpr int KR = 32 * KS;                // padded rank
  constexpr int STG = (KR * 8 + NT - 1) / NT;  // 16-byte W2 pieces per thread per tile
  constexpr int kBuf = KR * kLdsRow;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int row = blockIdx.y * 16 * NW + wave * 16 + n;  // this lane's row
  const int rowc = min(row, R - 1);

  // round t covers tiles t*G .. t*G + G-1 (G workgroups side by side: one
  // contiguous span of every W2 and base row); workgroup w takes slot
  // (w + 3t) mod G of it, so its tiles alternate in address parity (a fixed
  // slot leaves half the workgroups on odd 128-byte lines only, which stream
  // measurably slower)
  const int G = (int)gridDim.x;
  const int ntiles_all = (V + kTileCols - 1) / kTileCols;
  auto slot = [&](int t) -> int { return (int)(((int64_t)blockIdx.x + 3 * (int64_t)t) % G); };
  const int full = ntiles_all / G;
  const int ntile = full + (slot(full) < ntiles_all - full * G ? 1 : 0);
  auto tile_col = [&](int t) -> int64_t { return ((int64_t)t * G + slot(t)) * kTileCols; };

  // ---- E^T operands: rank 32kk + 8g .. +7 of W1[prev(row)]
  u32x4 eb[KS];
  auto gather_e = [&](int pv) {
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const int k = kk * 32 + g * 8;
      u32x4 v;
      if constexpr (EB) {
        const f32x4* ep = (const f32x4*)(ebuf + ((int64_t)rowc * gamma + step) * r + min(k, r - 8));
        const f32x4 x0 = ep[0], x1 = ep[1];
        v = u32x4{pack_bf16x2(x0[0], x0[1]), pack_bf16x2(x0[2], x0[3]), pack_bf16x2(x1[0], x1[1]),
                  pack_bf16x2(x1[2], x1[3])};
      } else {
        v = *(const u32x4*)(w1 + (int64_t)pv * r + min(k, r - 8));
      }
      eb[kk] = (row < R && k < r) ? v : u32x4{0u, 0u, 0u, 0u};
    }
  };

  // ---- staging: W2 piece i of thread t is rank row (t + i*NT) / 8, octet
  //      (t + i*NT) % 8 of the tile; base: the lane's row, columns 16j + 4g
  struct Set {
    u32x4 w[STG];
    f32x4 b[4];
  };
  auto load_set = [&](int t, Set& st) {
    const int64_t tc = tile_col(max(min(t, ntile - 1), 0));
#pragma unroll
    for (int i = 0; i < STG; ++i) {
      const int pc = threadIdx.x + i * NT;
      const int k = pc >> 3, oc = pc & 7;
      const int64_t col = tc + oc * 8;
      const u32x4 v = *(const u32x4*)(w2 + (int64_t)min(k, r - 1) * V + min(col, (int64_t)V - 8));
      st.w[i] = (k < r && col < V) ? v : u32x4{0u, 0u, 0u, 0u};
    }
    // the base logits are read once: non-temporal loads, so that they do not push the W2 tiles
    // (read again by the next step) out of the caches
    if constexpr (FL) {
      // whole 128-byte lines: load j covers rows 4j + lane/16 of the wave's 16,
      // 16-byte chunk lane % 16 of the tile's 256 bytes per row
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rj = min(blockIdx.y * 16 * NW + wave * 16 + 4 * j + (lane >> 4), R - 1);
        st.b[j] = __builtin_nontemporal_load((const f32x4*)(base + ((int64_t)rj * gamma + step) * V + min(tc + 4 * (lane & 15), (int64_t)V - 4)));
      }
    } else {
      const float* brow = base + ((int64_t)rowc * gamma + step) * V;
#pragma unroll
      for (int j = 0; j < 4; ++j) st.b[j] = __builtin_nontemporal_load((const f32x4*)(brow + min(tc + 16 * j + 4 * g, (int64_t)V - 4)));
    }
  };
  auto store_w2 = [&](unsigned char* bufp, const Set& st) {
#pragma unroll
    for (int i = 0; i < STG; ++i) {
      const int pc = threadIdx.x + i * NT;
      if (KR * 8 % NT == 0 || pc < KR * 8) *(u32x4*)(bufp + (pc >> 3) * kLdsRow + (pc & 7) * 16) = st.w[i];
    }
  };

  float best_z = -INFINITY;
  uint32_t best_v = 0xffffffffu;

  // A operand of product j, rank step kk: the lane (as source of the
  // transposing read) addresses rank row 32kk + 8g + s/4 (+4 for the second
  // read) and columns 16j + 4(s mod 4) .. +3, s = lane mod 16; it receives
  // W2[32kk + 8g + e][16j + s] for e = 0..7.
  typedef short i16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const uint32_t a_lane = (uint32_t)(8 * g + n / 4) * kLdsRow + 8 * (n % 4);
  // FL: the lane's base logits (row n, columns 16j + 4g .. +3) arrive spread
  // over the wave and are regathered through the wave's own 4 KB of LDS (row
  // q, 16-byte chunk c stored at chunk c ^ q: both passes conflict-free)
  unsigned char* const wave_lds = smem + 2 * kBuf + wave * 4096;
  auto regather = [&](const Set& in, f32x4* b) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int q = 4 * j + (lane >> 4), c = lane & 15;
      *(f32x4*)(wave_lds + q * 256 + ((c ^ q) << 4)) = in.b[j];
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = *(const f32x4*)(wave_lds + n * 256 + (((4 * j + g) ^ n) << 4));
  };
  auto compute_tile = [&](int t, const unsigned char* cur, const Set& st) {
    f32x4 bl[4];
    if constexpr (FL) {
      regather(st, bl);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) bl[j] = st.b[j];
    }
    f32x4 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const unsigned char* ap = cur + a_lane + kk * 32 * kLdsRow + 32 * j;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)ap);
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(ap + 4 * kLdsRow));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        acc[j] = mfma16x16x32(u32x4{l2.x, l2.y, h2.x, h2.y}, eb[kk], acc[j]);
      }
    }
    // epilogue: lane owns row `row`, columns v0 + 16j .. +3
    const int64_t v0 = tile_col(t) + 4 * g;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t vj = v0 + 16 * j;
      const bool colok = t < ntile && vj < V;
      f32x4 l = acc[j] + bl[j];
      if constexpr (SC) {
#pragma unroll
        for (int e = 0; e < 4; ++e) l[e] = tanhf(l[e] * invT) / invT;
      }
      if (step_logits && colok && row < R)
        *(f32x4*)(step_logits + ((int64_t)row * gamma + step) * V + vj) = l;
      f32x4 z = l;
      if (!greedy) {
        const u32x4 x = philox4x32_10(u32x4{(uint32_t)(vj >> 2), (uint32_t)step, (uint32_t)row, 0u},
                                      seed_lo, seed_hi);
#pragma unroll
        for (int e = 0; e < 4; ++e) z[e] = fmaf(l[e], invT, gumbel_from_bits(x[e]));
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool better = colok && z[e] > best_z;
        best_z = better ? z[e] : best_z;
        best_v = better ? (uint32_t)(vj + e) : best_v;
      }
    }
  };

  // prologue: tile 0's loads, then the dependent chain (previous keys, then
  // the W1 rows they select), then the other sets: tile 0 arrives while the
  // chain runs and the chain's reads do not queue behind the bulk prefetch
  Set sets[NS];
  load_set(0, sets[0]);
  if constexpr (EB) {
    gather_e(0);
  } else {
    const int pv = decode_prev(keys_prev, first_prev, rowc, R, V,
                               blockIdx.x == 0 && g == 0 && row < R ? status : nullptr);
    gather_e(pv);
  }
#pragma unroll
  for (int q = 1; q < NS; ++q) load_set(q, sets[q]);
  store_w2(smem, sets[0]);
  __syncthreads();
  // iteration t: compute tile t (LDS buffer t & 1, base from its set), load
  // tile t + NS into that set, move tile t + 1's W2 into the other buffer
  // (unrolled by NS so every set has fixed registers)
  for (int t0 = 0; t0 < ntile; t0 += NS) {
#pragma unroll
    for (int q = 0; q < NS; ++q) {
      const int t = t0 + q;
      if (t >= ntile) break;
      compute_tile(t, smem + (t & 1) * kBuf, sets[q]);
      load_set(t + NS, sets[q]);
      store_w2(smem + ((t + 1) & 1) * kBuf, sets[(q + 1) % NS]);
      __syncthreads();
    }
  }

  // ---- fold: the 4 lanes sharing a row, then the grid
  uint64_t key = best_v == 0xffffffffu ? 0ull : argmax_key(best_z, best_v);
#pragma unroll
  for (int m = 16; m < 64; m <<= 1) {
    const uint64_t o = shfl_xor_u64(key, m);
    key = o > key ? o : key;
  }
  if (g == 0 && key && row < R) fold_key_global(keys_out, row, R, key);
}

// ------------------------------------------------------------- vector path
// float32 (or unaligned bf16) weights: one thread per quad of columns,
// RC rows per pass (16, or 4 when 16-row chunks would leave most compute
// units idle) with E in LDS, fp32 FMAs.
constexpr int kRowChunk = 16;
constexpr int kVThreads = 64;  // one wave per workgroup

// One wave per (RC-row chunk, run of column quads): E = the chunk's rank-r
// rows, transposed into LDS ([k][RC rows]) so that each rank step reads the
// RC values with RC / 4 broadcast reads; every lane owns one quad of columns
// at a time and accumulates its RC x 4 products in registers.
template <bool kBf16W, bool SC = false, bool EB = false, int RC = kRowChunk>
__global__ __launch_bounds__(kVThreads) void markov_step_valu(
    const float* __restrict__ base, const void* __restrict__ w1v, const float* __restrict__ ebuf,
    const void* __restrict__ w2v,
    const int32_t* __restrict__ first_prev, const uint64_t* __restrict__ keys_prev,
    uint64_t* __restrict__ keys_out, float* __restrict__ step_logits, int R, int gamma, int V,
    int r, int step, float invT, int greedy, uint32_t seed_lo, uint32_t seed_hi,
    int32_t* __restrict__ status) {
  extern __shared__ __align__(16) unsigned char smem[];
  float* Et = (float*)smem;  // [r][RC]
  __shared__ int prev_tok[RC];
  auto w1 = [&](int64_t i) -> float {
    return kBf16W ? __uint_as_float((uint32_t)((const uint16_t*)w1v)[i] << 16) : ((const float*)w1v)[i];
  };
  auto w2 = [&](int64_t i) -> float {
    return kBf16W ? __uint_as_float((uint32_t)((const uint16_t*)w2v)[i] << 16) : ((const float*)w2v)[i];
  };
  const int row0 = blockIdx.y * RC;
  if (!EB && threadIdx.x < RC) {  // the chunk's previous tokens, decoded once
    const int row = row0 + threadIdx.x;
    prev_tok[threadIdx.x] =
        row < R ? decode_prev(keys_prev, first_prev, row, R, V, blockIdx.x == 0 ? status : nullptr) : 0;
  }
  __syncthreads();
  for (int c = threadIdx.x; c < RC * r; c += kVThreads) {
    const int rr = c / r, k = c % r, row = row0 + rr;
    float v = 0.f;
    if (row < R) {
      if constexpr (EB) v = ebuf[((int64_t)row * gamma + step) * r + k];
      else v = w1((int64_t)prev_tok[rr] * r + k);
    }
    Et[k * RC + rr] = v;
  }
  __syncthreads();

  const int64_t nq = (V + 3) / 4;
  float best_z[RC];
  uint32_t best_v[RC];
#pragma unroll
  for (int i = 0; i < RC; ++i) { best_z[i] = -INFINITY; best_v[i] = 0xffffffffu; }
  for (int64_t q = (int64_t)blockIdx.x * kVThreads + threadIdx.x; q < nq; q += (int64_t)gridDim.x * kVThreads) {
    const int64_t v0 = q * 4;
    float acc[RC][4];
#pragma unroll
    for (int i = 0; i < RC; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
    constexpr int kKB = 8;  // rank steps whose W2 loads go out together
    for (int k0 = 0; k0 < r; k0 += kKB) {
      float w[kKB][4];
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          w[kb][j] = (k0 + kb < r && v0 + j < V) ? w2((int64_t)(k0 + kb) * V + v0 + j) : 0.f;
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb) {
        if (k0 + kb >= r) break;
        const f32x4* e4 = (const f32x4*)(Et + (k0 + kb) * RC);
#pragma unroll
        for (int i4 = 0; i4 < RC / 4; ++i4) {
          const f32x4 e = e4[i4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            acc[4 * i4 + 0][j] = fmaf(e[0], w[kb][j], acc[4 * i4 + 0][j]);
            acc[4 * i4 + 1][j] = fmaf(e[1], w[kb][j], acc[4 * i4 + 1][j]);
            acc[4 * i4 + 2][j] = fmaf(e[2], w[kb][j], acc[4 * i4 + 2][j]);
            acc[4 * i4 + 3][j] = fmaf(e[3], w[kb][j], acc[4 * i4 + 3][j]);
          }
        }
      }
    }
    float bl[RC][4];  // the chunk's base logits, all loads in flight together
#pragma unroll
    for (int i = 0; i < RC; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bl[i][j] = (row0 + i < R && v0 + j < V) ? base[((int64_t)(row0 + i) * gamma + step) * V + v0 + j] : 0.f;
#pragma unroll
    for (int i = 0; i < RC; ++i) {
      const int row = row0 + i;
      if (row >= R) break;
      u32x4 xs = u32x4{0u, 0u, 0u, 0u};
      if (!greedy) xs = philox4x32_10(u32x4{(uint32_t)q, (uint32_t)step, (uint32_t)row, 0u}, seed_lo, seed_hi);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t v = v0 + j;
        if (v >= V) break;
        const int64_t off = ((int64_t)row * gamma + step) * V + v;
        float l = bl[i][j] + acc[i][j];
        if constexpr (SC) l = tanhf(l * invT) / invT;
        if (step_logits) step_logits[off] = l;
        const float z = greedy ? l : fmaf(l, invT, gumbel_from_bits(xs[j]));
        if (z > best_z[i]) { best_z[i] = z; best_v[i] = (uint32_t)v; }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < RC; ++i) {
    uint64_t key = best_v[i] == 0xffffffffu ? 0ull : argmax_key(best_z[i], best_v[i]);
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const uint64_t o = shfl_xor_u64(key, m);
      key = o > key ? o : key;
    }
    const int row = row0 + i;
    if (threadIdx.x == 0 && row < R && key) fold_key_global(keys_out, row, R, key);
  }
}

__global__ void zero_u64_kernel(uint64_t* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0ull;
}

__global__ void finalize_tokens_kernel(const uint64_t* __restrict__ keys, int32_t* __restrict__ tokens,
                                       int R, int gamma, int V, int32_t* status) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // over [R, gamma]
  if (i >= (int64_t)R * gamma) return;
  const int row = (int)(i / gamma), step = (int)(i % gamma);
  uint32_t t = argmax_key_index(read_key(keys + (int64_t)step * keys_per_step(R), row, R));
  if (t >= (uint32_t)V) { status_or(status, DSPARK_STATUS_BAD_TOKEN); t = 0; }
  tokens[i] = (int32_t)t;
}

int cu_count() {
  static std::atomic<int> cache[64];  // per device, 0 = unknown
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (dev >= 0 && dev < 64 && (cus = cache[dev].load(std::memory_order_relaxed)) > 0) return cus;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  if (dev >= 0 && dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// Raise a kernel's dynamic-LDS limit once per process (the call costs tens
// of microseconds of host time, far more than a step's launch).
template <typename K>
hipError_t allow_lds_once(K kern, size_t bytes) {
  static KeyedCache<size_t> done;
  size_t have = 0;
  if (done.find(0, (const void*)kern, have) && have >= bytes) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)bytes);
  if (e == hipSuccess) done.put(0, (const void*)kern, bytes);
  return e;
}

template <int NW, int KS, int NS, bool FL, bool SC, bool EB>
hipError_t launch_mfma(int grid_x, int grid_y, hipStream_t s, const float* base, const uint16_t* w1,
                       const float* ebuf, const uint16_t* w2, const int32_t* first_prev, const uint64_t* kp,
                       uint64_t* ko, float* step_logits, int R, int gamma, int V, int r, int step,
                       float invT, int greedy, uint32_t slo, uint32_t shi, int32_t* st) {
  (void)r;
  const size_t shm = (size_t)2 * 32 * KS * kLdsRow + (FL ? (size_t)NW * 4096 : 0);
  auto kern = markov_step_mfma<NW, KS, NS, FL, SC, EB>;
  hipError_t e = allow_lds_once(kern, shm);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid_x, grid_y), dim3(64 * NW), shm, s, base, w1, ebuf, w2, first_prev,
                     kp, ko, step_logits, R, gamma, V, r, step, invT, greedy, slo, shi, st);
  return hipGetLastError();
}


// One step over R rows: the MFMA kernel for bf16 weights in aligned buffers
// (up to 128 rows per workgroup, 8 waves, one compute unit each; up to 64
// rows use 4 waves and two workgroups per compute unit), else the vector
// kernel.
template <bool SC, bool EB = false>
hipError_t launch_step(bool mfma_ok, bool bf, int cus, hipStream_t s, const float* base, const void* w1,
                       const float* ebuf, const void* w2, const int32_t* first_prev, const uint64_t* kp, uint64_t* ko,
                       float* step_logits, int R, int gamma, int V, int r, int step, float invT,
                       int greedy, uint32_t slo, uint32_t shi, int32_t* st) {
  if (mfma_ok) {
    const bool wide = R > 64;
    const int rows_per = wide ? 128 : 64;
    const int gy = (R + rows_per - 1) / rows_per;
    int gx = wide ? cus : 2 * cus;
    const int64_t tiles = (V + 63) / 64;
    if (gx > tiles) gx = (int)tiles;
    if (gx < 1) gx = 1;
    const uint16_t *a = (const uint16_t*)w1, *b = (const uint16_t*)w2;
    if (wide)
      return r <= 256 ? launch_mfma<8, 8, 2, true, SC, EB>(gx, gy, s, base, a, ebuf, b, first_prev, kp, ko, step_logits, R, gamma, V, r, step, invT, greedy, slo, shi, st)
                      : launch_mfma<8, 16, 2, false, SC, EB>(gx, gy, s, base, a, ebuf, b, first_prev, kp, ko, step_logits, R, gamma, V, r, step, invT, greedy, slo, shi, st);
    return r <= 256 ? launch_mfma<4, 8, 2, false, SC, EB>(gx, gy, s, base, a, ebuf, b, first_prev, kp, ko, step_logits, R, gamma, V, r, step, invT, greedy, slo, shi, st)
                    : launch_mfma<4, 16, 2, false, SC, EB>(gx, gy, s, base, a, ebuf, b, first_prev, kp, ko, step_logits, R, gamma, V, r, step, invT, greedy, slo, shi, st);
  }
  int gx = 4 * cus;
  const int64_t quads = (V + 3) / 4;
  if ((int64_t)gx * kVThreads > quads) gx = (int)((quads + kVThreads - 1) / kVThreads);
  if (gx < 1) gx = 1;
  // small shapes (a few dozen single-wave workgroups at 16 rows each) take 4-row chunks:
  // four times the workgroups, a quarter of each lane's chain
  const bool narrow = (int64_t)gx * ((R + kRowChunk - 1) / kRowChunk) < cus;
  const int rc = narrow ? 4 : kRowChunk;
  const int gy = (R + rc - 1) / rc;
  const size_t shm = (size_t)rc * r * 4;
  auto go = [&](auto kern) {
    (void)allow_lds_once(kern, shm);
    hipLaunchKernelGGL(kern, dim3(gx, gy), dim3(kVThreads), shm, s, base, w1, ebuf, w2, first_prev, kp, ko,
                       step_logits, R, gamma, V, r, step, invT, greedy, slo, shi, st);
  };
  if (bf) {
    if (narrow) go(markov_step_valu<true, SC, EB, 4>);
    else go(markov_step_valu<true, SC, EB>);
  } else {
    if (narrow) go(markov_step_valu<false, SC, EB, 4>);
    else go(markov_step_valu<false, SC, EB>);
  }
  return hipGetLastError();
}

}  // namespace

namespace dspark {

hipError_t markov_step_embedded(const float* base, const float* ebuf, const void* w2, int wdtype,
                                uint64_t* keys_out, float* step_logits, int R, int gamma, int V, int r, int step,
                                float softcap, float temperature, uint64_t seed, hipStream_t s) {
  const int cus = cu_count();
  if (cus <= 0) return hipErrorInvalidDevice;
  const bool bf = wdtype == DSPARK_BF16;
  const bool mfma_ok = bf && V % 8 == 0 && r % 8 == 0 && r <= 512 && (uintptr_t)w2 % 16 == 0 &&
                       (uintptr_t)ebuf % 16 == 0 && (uintptr_t)base % 16 == 0 &&
                       (!step_logits || (uintptr_t)step_logits % 16 == 0);
  const uint32_t slo = (uint32_t)seed, shi = (uint32_t)(seed >> 32);
  if (softcap > 0.f)
    return launch_step<true, true>(mfma_ok, bf, cus, s, base, nullptr, ebuf, w2, nullptr, nullptr, keys_out,
                                   step_logits, R, gamma, V, r, step, 1.f / softcap, 1, 0u, 0u, nullptr);
  const int greedy = temperature == 0.f;
  return launch_step<false, true>(mfma_ok, bf, cus, s, base, nullptr, ebuf, w2, nullptr, nullptr, keys_out,
                                  step_logits, R, gamma, V, r, step, greedy ? 1.f : 1.f / temperature, greedy,
                                  slo, shi, nullptr);
}

hipError_t markov_zero_keys(uint64_t* keys, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_u64_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, keys, n);
  return hipGetLastError();
}

hipError_t markov_finalize_tokens(const uint64_t* keys, int32_t* tokens, int R, int gamma, int V,
                                  int32_t* status, hipStream_t s) {
  const int64_t n = (int64_t)R * gamma;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(finalize_tokens_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, keys, tokens,
                     R, gamma, V, status);
  return hipGetLastError();
}

}  // namespace dspark

extern "C" size_t dspark_markov_sample_workspace_bytes(int R, int gamma, int V, int r, int wdtype) {
  (void)V; (void)r; (void)wdtype;
  if (R <= 0 || gamma <= 0) return 0;
  return (size_t)gamma * keys_per_step(R) * sizeof(uint64_t);
}

namespace {

// Host-side checks shared by both sampler entry points; 0 = go on, 1 = done
// (nothing to do), else the status to return.
int markov_sample_check(const char* who, const float* base_logits, const void* w1, const void* w2,
                        const int32_t* first_prev, const int32_t* tokens, int R, int gamma, int V, int r,
                        int wdtype, float temperature) {
  using namespace dspark_host;
  if (R < 0 || gamma < 0) return fail(DSPARK_ERR_INVALID_ARG, "%s: negative dimension", who);
  if (V < 1 || r < 1 || r > 1024)
    return fail(DSPARK_ERR_INVALID_ARG, "%s: need V >= 1 and 1 <= r <= 1024 (V=%d r=%d)", who, V, r);
  if (gamma > 1024) return fail(DSPARK_ERR_INVALID_ARG, "%s: gamma > 1024", who);
  if (wdtype != DSPARK_BF16 && wdtype != DSPARK_F32)
    return fail(DSPARK_ERR_INVALID_ARG, "%s: unknown wdtype %d", who, wdtype);
  if (!(temperature >= 0.f) || temperature == INFINITY)
    return fail(DSPARK_ERR_INVALID_ARG, "%s: temperature must be finite and >= 0", who);
  if ((int64_t)R * gamma == 0) {
    ok();
    return 1;
  }
  if (!base_logits || !w1 || !w2 || !first_prev || !tokens)
    return fail(DSPARK_ERR_INVALID_ARG, "%s: null required pointer", who);
  return 0;
}

// The sampler proper over a key buffer of dspark_markov_sample_workspace_bytes.
int markov_sample_run(const float* base_logits, const void* w1, const void* w2, const int32_t* first_prev,
                      int32_t* tokens, float* step_logits, int R, int gamma, int V, int r, int wdtype,
                      float temperature, uint64_t seed, uint64_t* keys, int32_t* dev_status, hipStream_t s) {
  using namespace dspark_host;
  const int64_t nk = (int64_t)gamma * keys_per_step(R);
  hipLaunchKernelGGL(zero_u64_kernel, dim3((unsigned)((nk + 255) / 256)), dim3(256), 0, s, keys, nk);
  const int greedy = temperature == 0.f;
  const float invT = greedy ? 1.f : 1.f / temperature;
  const uint32_t slo = (uint32_t)seed, shi = (uint32_t)(seed >> 32);
  const int cus = cu_count();
  if (cus <= 0) return fail(DSPARK_ERR_HIP, "markov_sample: device query failed");

  const bool bf = wdtype == DSPARK_BF16;
  // up to 128 rows with bf16 weights: every step in one persistent launch with W2 held in
  // registers (markov_round.hip); otherwise one launch per step
  if (bf && markov_round_eligible(R, gamma, V, r, base_logits, w1, w2, step_logits)) {
    const hipError_t e = markov_round_launch(base_logits, (const uint16_t*)w1, (const uint16_t*)w2, first_prev,
                                             tokens, step_logits, R, gamma, V, r, invT, greedy, slo, shi, keys,
                                             wait_limit(), dev_status, s);
    if (e == hipSuccess) return check_launch("markov_sample");
    if (e != hipErrorNotSupported)
      return fail(DSPARK_ERR_HIP, "markov_sample (one launch): %s", hipGetErrorString(e));
  }
  const bool mfma_ok = bf && V % 8 == 0 && r % 8 == 0 && r <= 512 && (uintptr_t)w1 % 16 == 0 &&
                       (uintptr_t)w2 % 16 == 0 && (uintptr_t)base_logits % 16 == 0 &&
                       (!step_logits || (uintptr_t)step_logits % 16 == 0);
  for (int step = 0; step < gamma; ++step) {
    const uint64_t* kp = step == 0 ? nullptr : keys + (int64_t)(step - 1) * keys_per_step(R);
    uint64_t* ko = keys + (int64_t)step * keys_per_step(R);
    const hipError_t e = launch_step<false>(mfma_ok, bf, cus, s, base_logits, w1, nullptr, w2, first_prev, kp, ko,
                                            step_logits, R, gamma, V, r, step, invT, greedy, slo, shi,
                                            dev_status);
    if (e != hipSuccess) return fail(DSPARK_ERR_HIP, "markov_sample step %d: %s", step, hipGetErrorString(e));
  }
  const int64_t ntok = (int64_t)R * gamma;
  hipLaunchKernelGGL(finalize_tokens_kernel, dim3((unsigned)((ntok + 255) / 256)), dim3(256), 0, s, keys,
                     tokens, R, gamma, V, dev_status);
  return check_launch("markov_sample");
}

}  // namespace

extern "C" int dspark_markov_sample(const float* base_logits, const void* w1, const void* w2,
                                   const int32_t* first_prev, int32_t* tokens, float* step_logits,
                                   int R, int gamma, int V, int r, int wdtype, float temperature,
                                   uint64_t seed, void* ws, size_t ws_bytes, int32_t* dev_status,
                                   void* stream) {
  using namespace dspark_host;
  const int c = markov_sample_check("markov_sample", base_logits, w1, w2, first_prev, tokens, R, gamma, V, r,
                                    wdtype, temperature);
  if (c != 0) return c == 1 ? DSPARK_OK : c;
  const size_t need = dspark_markov_sample_workspace_bytes(R, gamma, V, r, wdtype);
  if (ws_bytes < need || !ws)
    return fail(DSPARK_ERR_WORKSPACE, "markov_sample: workspace %zu bytes < %zu", ws_bytes, need);
  if ((uintptr_t)ws % 8) return fail(DSPARK_ERR_INVALID_ARG, "markov_sample: workspace not 8-byte aligned");
  return markov_sample_run(base_logits, w1, w2, first_prev, tokens, step_logits, R, gamma, V, r, wdtype,
                           temperature, seed, (uint64_t*)ws, dev_status, (hipStream_t)stream);
}

// Allocation-free variant: the key buffer is a fixed array in device memory
// (one copy per device, alive until the process ends).  In host code the
// array's name only stands in for it; its device address is looked up once
// per device and only that address is passed to kernels.
static __device__ __align__(256) uint64_t scratch[DSPARK_NOALLOC_SCRATCH_BYTES / sizeof(uint64_t)];

namespace {

uint64_t* noalloc_scratch(int* err_dev) {
  static std::atomic<void*> addr[64];  // per device, null = not looked up yet
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    *err_dev = dev;
    return nullptr;
  }
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p) return (uint64_t*)p;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
    *err_dev = dev;
    return nullptr;
  }
  addr[dev].store(p, std::memory_order_release);
  return (uint64_t*)p;
}

}  // namespace

extern "C" int dspark_markov_sample_noalloc(const float* base_logits, const void* w1, const void* w2,
                                           const int32_t* first_prev, int32_t* tokens, float* step_logits,
                                           int R, int gamma, int V, int r, int wdtype, float temperature,
                                           uint64_t seed, int32_t* dev_status, void* stream) {
  using namespace dspark_host;
  const int c = markov_sample_check("markov_sample_noalloc", base_logits, w1, w2, first_prev, tokens, R, gamma,
                                    V, r, wdtype, temperature);
  if (c != 0) return c == 1 ? DSPARK_OK : c;
  const size_t need = dspark_markov_sample_workspace_bytes(R, gamma, V, r, wdtype);
  if (need > DSPARK_NOALLOC_SCRATCH_BYTES)
    return fail(DSPARK_ERR_WORKSPACE,
                "markov_sample_noalloc: R=%d, gamma=%d need %zu bytes of scratch, above the fixed %zu "
                "(use dspark_markov_sample with a workspace)",
                R, gamma, need, (size_t)DSPARK_NOALLOC_SCRATCH_BYTES);
  int dev = -1;
  uint64_t* keys = noalloc_scratch(&dev);
  if (!keys) return fail(DSPARK_ERR_HIP, "markov_sample_noalloc: no scratch address on device %d", dev);
  return markov_sample_run(base_logits, w1, w2, first_prev, tokens, step_logits, R, gamma, V, r, wdtype,
                           temperature, seed, keys, dev_status, (hipStream_t)stream);
}

// Teacher-forced block logits (page 1 §3.7, apply_block_logits in training;
// page 4 §3.3): every row takes its bias from its own given previous token,
// so the whole block is one step of the kernels above over all N rows (one
// pass over W2 per 128-row group), with the base add, the optional soft cap
// and the logit store fused into the tile epilogue.  The argmax fold of that
// step gives each row's greedy token for free.
extern "C" size_t dspark_markov_block_logits_workspace_bytes(int N, int V, int r, int wdtype) {
  return dspark_markov_sample_workspace_bytes(N, 1, V, r, wdtype);
}

extern "C" int dspark_markov_block_logits(const float* base_logits, const void* w1, const void* w2,
                                          const int32_t* prev, float* logits, int32_t* argmax_tokens,
                                          int N, int V, int r, int wdtype, float softcap, void* ws,
                                          size_t ws_bytes, int32_t* dev_status, void* stream) {
  using namespace dspark_host;
  if (N < 0) return fail(DSPARK_ERR_INVALID_ARG, "markov_block_logits: negative dimension");
  if (V < 1 || r < 1 || r > 1024)
    return fail(DSPARK_ERR_INVALID_ARG, "markov_block_logits: need V >= 1 and 1 <= r <= 1024 (V=%d r=%d)", V, r);
  if (wdtype != DSPARK_BF16 && wdtype != DSPARK_F32)
    return fail(DSPARK_ERR_INVALID_ARG, "markov_block_logits: unknown wdtype %d", wdtype);
  if (!(softcap >= 0.f) || softcap == INFINITY)
    return fail(DSPARK_ERR_INVALID_ARG, "markov_block_logits: softcap must be finite and >= 0");
  if (N == 0) return ok();
  if (!base_logits || !w1 || !w2 || !prev || !logits)
    return fail(DSPARK_ERR_INVALID_ARG, "markov_block_logits: null required pointer");
  const size_t need = dspark_markov_block_logits_workspace_bytes(N, V, r, wdtype);
  if (ws_bytes < need || !ws)
    return fail(DSPARK_ERR_WORKSPACE, "markov_block_logits: workspace %zu bytes < %zu", ws_bytes, need);
  if ((uintptr_t)ws % 8) return fail(DSPARK_ERR_INVALID_ARG, "markov_block_logits: workspace not 8-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  uint64_t* keys = (uint64_t*)ws;
  const int64_t nk = keys_per_step(N);
  hipLaunchKernelGGL(zero_u64_kernel, dim3((unsigned)((nk + 255) / 256)), dim3(256), 0, s, keys, nk);
  const int cus = cu_count();
  if (cus <= 0) return fail(DSPARK_ERR_HIP, "markov_block_logits: device query failed");
  const bool bf = wdtype == DSPARK_BF16;
  // bf16 weights: one launch over all rows with W2 held in registers (markov_round.hip)
  if (bf && markov_rows_eligible(N, V, r, base_logits, w1, w2, logits)) {
    const hipError_t e = markov_rows_launch(base_logits, (const uint16_t*)w1, (const uint16_t*)w2, prev, logits, N, V,
                                            r, softcap, keys, dev_status, s);
    if (e != hipSuccess && e != hipErrorNotSupported)
      return fail(DSPARK_ERR_HIP, "markov_block_logits: %s", hipGetErrorString(e));
    if (e == hipSuccess) {
      if (argmax_tokens)
        hipLaunchKernelGGL(finalize_tokens_kernel, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, s, keys,
                           argmax_tokens, N, 1, V, dev_status);
      return check_launch("markov_block_logits");
    }
  }
  const bool mfma_ok = bf && V % 8 == 0 && r % 8 == 0 && r <= 512 && (uintptr_t)w1 % 16 == 0 &&
                       (uintptr_t)w2 % 16 == 0 && (uintptr_t)base_logits % 16 == 0 &&
                       (uintptr_t)logits % 16 == 0;
  // greedy, prev from the caller (no previous keys); with a soft cap the
  // temperature slot carries 1 / c
  const hipError_t e =
      softcap > 0.f
          ? launch_step<true>(mfma_ok, bf, cus, s, base_logits, w1, nullptr, w2, prev, nullptr, keys, logits, N, 1, V, r,
                              0, 1.f / softcap, 1, 0u, 0u, dev_status)
          : launch_step<false>(mfma_ok, bf, cus, s, base_logits, w1, nullptr, w2, prev, nullptr, keys, logits, N, 1, V,
                               r, 0, 1.f, 1, 0u, 0u, dev_status);
  if (e != hipSuccess) return fail(DSPARK_ERR_HIP, "markov_block_logits: %s", hipGetErrorString(e));
  if (argmax_tokens)
    hipLaunchKernelGGL(finalize_tokens_kernel, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, s, keys,
                       argmax_tokens, N, 1, V, dev_status);
  return check_launch("markov_block_logits");
}
