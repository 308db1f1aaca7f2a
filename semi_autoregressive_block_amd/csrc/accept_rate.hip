// TV-distance accept rate (page 1, "03 · DSpark 建模", §3.9, the paper's
// Eq. 8; page 2 §3.5 / §3.8.3) and tau (page 1 §3.10).
//
//   accept = clamp(1 - 1/2 sum_v |p_v - q_v|, 0, 1),  p = softmax(draft), q = softmax(target)
//
// computed through the equivalent form 1 - TV(p, q) = sum_v min(p_v, q_v)
// (valid because both distributions sum to one), which needs no absolute
// value and lets each workgroup fold its slice into one partial sum.
//
// HBM-bound design for gfx950: a row (2 x V logits) is split over a cluster of
// G workgroups that stay resident for the whole launch (cooperative grid).
// Each workgroup has three data waves and one exchange wave.  The data waves
// turn their slice of both tensors into exponentials 2^{x log2e - a}
// relative to the slice's own maximum a and sum them (pass one).  The row's
// normaliser needs every slice's (max, sum), which the exchange wave trades
// with the cluster through a few bytes of global memory; it issues no other
// loads, so its polls never queue behind the data waves' streaming loads.
// The exchange is pipelined: while it runs, the data waves park the row's
// exponentials in LDS and go on with pass one of the next row; pass two of
// a row (one fused multiply-add and one add per element pair through
// sum min = (sum p + sum q - sum |p - q|) / 2, no second exponential) runs
// one iteration later.  Cluster members may therefore drift
// apart by up to an iteration without stalling one another.  The next row's
// slice streams in (16-byte buffer loads; a row past the end reads through an
// empty buffer range, so the tail costs no traffic) while the current one is
// reduced.  Each workgroup writes its slice's share of sum_v min(p_v, q_v) to
// the workspace and a small kernel folds the G shares of a row in fixed
// order (deterministic results) into the accept rate and tau.
#include <stdlib.h>

#include <algorithm>
#include <atomic>

#include "cluster.h"
#include "common.h"
#include "host_cache.h"

using namespace dspark;
using namespace dspark::cluster;

namespace {

constexpr int kDataWaves = 3;
constexpr int kDataThreads = kDataWaves * kWave;  // threads that hold the row slice
constexpr int kThreads = kDataThreads + kWave;    // plus the exchange wave
constexpr int kVec = 4;                           // 16-byte vectors per data thread per tensor (a 24 KB
                                                  // slice of both tensors; three workgroups per CU)
constexpr int kChunkVec = kDataThreads * kVec;    // vectors of one tensor per workgroup and row
constexpr int kMaxG = 2 * kWave;                  // two cluster members per exchange lane


// bf16 (or float32) vector of the raw slice -> float32 values; lanes whose
// vector lies past the row end hold zeros (empty buffer range) and are made
// -inf, which drops them from the max and turns their exponentials into 0.
template <bool kBf16>
__device__ __forceinline__ void unpack(const u32x4& r, float* x, bool valid) {
  const uint32_t pad = valid ? 0u : 0xff800000u;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    if (kBf16) {
      x[2 * c] = __uint_as_float((r[c] << 16) | pad);
      x[2 * c + 1] = __uint_as_float((r[c] & 0xffff0000u) | pad);
    } else {
      x[c] = __uint_as_float(r[c] | pad);
    }
  }
}
template <bool kBf16>
__device__ __forceinline__ void unpack_fast(const u32x4& r, float* x) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    if (kBf16) {
      x[2 * c] = bf16lo(r[c]);
      x[2 * c + 1] = bf16hi(r[c]);
    } else {
      x[c] = __uint_as_float(r[c]);
    }
  }
}

template <bool kBf16>
struct Shape {
  static constexpr int kEl = kBf16 ? 8 : 4;  // elements per 16-byte vector
  static constexpr int kN = kVec * kEl;      // floats per data thread per tensor
  static constexpr int kPark = 2 * kN / 4;   // float4 slots per data thread (both tensors)
};

// Workspace: shares [rows][G] float | slots [clusters][2 parities][G] 16-byte words | error word.
template <bool kBf16>
__global__ __launch_bounds__(kThreads) void tv_cluster_kernel(
    const char* __restrict__ d, const char* __restrict__ t, float* __restrict__ share,
    int64_t rows, int V, int vec_per_row, int G, int nclusters,
    u32x4* __restrict__ slots, int32_t* __restrict__ err, unsigned spin_limit) {
  constexpr int kEl = Shape<kBf16>::kEl, kN = Shape<kBf16>::kN, kPark = Shape<kBf16>::kPark;
  __shared__ f32x4 park[kPark][kDataThreads];  // the previous row's exponentials
  __shared__ float red_max[2][2][kDataWaves], red_sum[2][2][kDataWaves], red_part[kDataWaves];
  __shared__ float glob[2][2];  // [parity of the row][draft, target]
  const int cl = blockIdx.x / G, g = blockIdx.x % G;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform role
  const uint32_t row_bytes = (uint32_t)V * (kBf16 ? 2u : 4u);
  u32x4* cslots = slots + (size_t)cl * 2 * G;
  const int64_t nk = (rows - cl + nclusters - 1) / nclusters;  // rows of this cluster (cl < rows)

  if (w < kDataWaves) {
    // ------------------------------------------------------------ data waves
    const int tid = threadIdx.x;
    const int vbase = g * kChunkVec;
    // slot i of this thread is vector vbase + i * kDataThreads + tid of the
    // row: one per-lane byte offset plus a per-slot scalar offset.  Vectors
    // past the row end fall outside the buffer range and read as zeros.
    const uint32_t voff = (uint32_t)(vbase + tid) * 16u;
    bool full[kVec];
#pragma unroll
    for (int i = 0; i < kVec; ++i) full[i] = vbase + (i + 1) * kDataThreads <= vec_per_row;  // uniform
    u32x4 rd[kVec], rt[kVec];
    auto issue = [&](int64_t row) {
      const bool in = row < rows;
      const int64_t off = (in ? row : 0) * (int64_t)row_bytes;
      const int nrec = in ? (int)row_bytes : 0;
      const __amdgpu_buffer_rsrc_t sd = __builtin_amdgcn_make_buffer_rsrc((void*)(d + off), 0, nrec, kRsrcWord3);
      const __amdgpu_buffer_rsrc_t st = __builtin_amdgcn_make_buffer_rsrc((void*)(t + off), 0, nrec, kRsrcWord3);
#pragma unroll
      for (int i = 0; i < kVec; ++i) {
        rd[i] = __builtin_amdgcn_raw_buffer_load_b128(sd, voff, i * kDataThreads * 16, kNonTemporal);
        rt[i] = __builtin_amdgcn_raw_buffer_load_b128(st, voff, i * kDataThreads * 16, kNonTemporal);
      }
    };
    issue(cl);
    float psd = 0.f, pst = 0.f;  // this wave's sums of the previous row's exponentials
    for (int64_t k = 0; k <= nk; ++k) {
      const int64_t row = cl + k * nclusters;
      const bool have = k < nk;  // iteration nk only finishes the last row
      const int par = (int)(k & 1);
      float xd[kN], xt[kN];
      float csd = 0.f, cst = 0.f;
      if (have) {
#pragma unroll
        for (int i = 0; i < kVec; ++i) {
          if (full[i]) {
            unpack_fast<kBf16>(rd[i], xd + i * kEl);
            unpack_fast<kBf16>(rt[i], xt + i * kEl);
          } else {
            const bool valid = vbase + i * kDataThreads + tid < vec_per_row;
            unpack<kBf16>(rd[i], xd + i * kEl, valid);
            unpack<kBf16>(rt[i], xt + i * kEl, valid);
          }
        }
        issue(row + nclusters);  // the next row streams in while this one is reduced
        float md = xd[0], mt = xt[0];
#pragma unroll
        for (int i = 1; i < kN; ++i) {
          md = vmax(md, xd[i]);
          mt = vmax(mt, xt[i]);
        }
        md = wave_max(md);
        mt = wave_max(mt);
        if (lane == 0) { red_max[par][0][w] = md; red_max[par][1][w] = mt; }
      }
      __syncthreads();  // A: slice maxima of row k; the partial sums of row k-2 are complete
      if (have) {
        const float mD = vmax(vmax(red_max[par][0][0], red_max[par][0][1]), red_max[par][0][2]);
        const float mT = vmax(vmax(red_max[par][1][0], red_max[par][1][1]), red_max[par][1][2]);
        const float aD = mD == -INFINITY ? 0.f : mD * kLog2e;
        const float aT = mT == -INFINITY ? 0.f : mT * kLog2e;
        float sd0 = 0.f, sd1 = 0.f, st0 = 0.f, st1 = 0.f;
#pragma unroll
        for (int i = 0; i < kN; i += 2) {
          xd[i] = exp2_fast(fmaf(xd[i], kLog2e, -aD));
          xd[i + 1] = exp2_fast(fmaf(xd[i + 1], kLog2e, -aD));
          xt[i] = exp2_fast(fmaf(xt[i], kLog2e, -aT));
          xt[i + 1] = exp2_fast(fmaf(xt[i + 1], kLog2e, -aT));
          sd0 += xd[i]; sd1 += xd[i + 1];
          st0 += xt[i]; st1 += xt[i + 1];
        }
        const float wsd = wave_sum(sd0 + sd1), wst = wave_sum(st0 + st1);
        if (lane == 0) { red_sum[par][0][w] = wsd; red_sum[par][1][w] = wst; }
        csd = wsd;
        cst = wst;
      }
      __syncthreads();  // B: sums of row k; the exchange wave has the offsets of row k-1
      if (k >= 1) {
        // pass two of row k-1 on its parked exponentials:
        // p_v = ed_v * 2^{eD}, q_v = et_v * 2^{eT}; the side with the smaller
        // exponent is scaled down (never up: no overflow, and 0 * c stays 0).
        // With u the unscaled side and v the scaled one,
        //   sum min(u, v) = (sum u + sum v - sum |u - v|) / 2,
        // where both sums are this wave's pass-one sums of the row: one fma
        // (|.| is a free source modifier of the add) and one add per pair.
        const float eD = uniform(glob[(k - 1) & 1][0]), eT = uniform(glob[(k - 1) & 1][1]);
        float p0 = 0.f, p1 = 0.f, su, sv;
        if (eD >= eT) {
          const float c = exp2_fast(eT - eD);
          su = psd;
          sv = pst * c;
#pragma unroll
          for (int j = 0; j < kN / 4; ++j) {
            const f32x4 a = park[j][tid], b = park[kN / 4 + j][tid];
            p0 += fabsf(fmaf(b[0], c, -a[0])); p1 += fabsf(fmaf(b[1], c, -a[1]));
            p0 += fabsf(fmaf(b[2], c, -a[2])); p1 += fabsf(fmaf(b[3], c, -a[3]));
          }
        } else {
          const float c = exp2_fast(eD - eT);
          su = pst;
          sv = psd * c;
#pragma unroll
          for (int j = 0; j < kN / 4; ++j) {
            const f32x4 a = park[j][tid], b = park[kN / 4 + j][tid];
            p0 += fabsf(fmaf(a[0], c, -b[0])); p1 += fabsf(fmaf(a[1], c, -b[1]));
            p0 += fabsf(fmaf(a[2], c, -b[2])); p1 += fabsf(fmaf(a[3], c, -b[3]));
          }
        }
        const float wp = 0.5f * ((su + sv) - wave_sum(p0 + p1));
        if (lane == 0) red_part[w] = wp;  // times 2^{max(eD, eT)}: applied by the exchange wave
      }
      psd = csd;
      pst = cst;
      if (have) {
#pragma unroll
        for (int j = 0; j < kN / 4; ++j) {
          park[j][tid] = f32x4{xd[4 * j], xd[4 * j + 1], xd[4 * j + 2], xd[4 * j + 3]};
          park[kN / 4 + j][tid] = f32x4{xt[4 * j], xt[4 * j + 1], xt[4 * j + 2], xt[4 * j + 3]};
        }
      }
    }
    __syncthreads();  // the last row's partial sums are complete
  } else {
    // --------------------------------------------------------- exchange wave
    // It also does every global store of the workgroup (published statistics
    // and shares), so that the data waves' waits on their streaming loads
    // never include a store acknowledgement.  Its short, latency-bound
    // sequence decides when the data waves may pass barrier B, so it issues
    // ahead of them on its SIMD.
    auto store_share = [&](int64_t kk) {  // share of the cluster's row kk, from red_part
      if (lane == 0) {
        const int pp = (int)(kk & 1);
        const float scale = exp2_fast(vmax(glob[pp][0], glob[pp][1]));  // NaN stays NaN
        share[(cl + kk * nclusters) * G + g] = ((red_part[0] + red_part[1]) + red_part[2]) * scale;
      }
    };
    __builtin_amdgcn_s_setprio(3);
    bool ok = true;  // after one timed-out wait this lane stops waiting
    for (int64_t k = 0; k <= nk; ++k) {
      unsigned n = 0;  // polls of this lane for this row, for the bound
      // offsets of row k-1: the cluster publishes its slice statistics after
      // its barrier B; lane l gathers members l and l + 64 (after barrier A)
      const int par = (int)((k - 1) & 1);
      const uint32_t epoch = (uint32_t)k;
      float ad[2] = {-INFINITY, -INFINITY}, sd[2] = {0.f, 0.f};
      float at[2] = {-INFINITY, -INFINITY}, st[2] = {0.f, 0.f};
      bool got[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int j = lane + h * kWave;
        got[h] = k == 0 || j >= G || j == g;  // nothing to fetch
      }
      auto poll = [&]() {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          if (!got[h]) {
            const u32x4 v = peek(cslots + (size_t)par * G + lane + h * kWave);
            if (fresh(v, epoch)) {
              ad[h] = __uint_as_float(v[0]); sd[h] = __uint_as_float(v[1]);
              at[h] = __uint_as_float(v[2]); st[h] = __uint_as_float(v[3]);
              got[h] = true;
            } else if (!ok || ++n > spin_limit) {
              if (ok) atomicOr(err, DSPARK_STATUS_WAIT_TIMEOUT);
              ok = false;
              got[h] = true;  // give up on this member: the row is poisoned below
            }
          }
        }
      };
      __syncthreads();  // A
      while (!__all(got[0] && got[1])) {
        poll();
        if (!__all(got[0] && got[1])) __builtin_amdgcn_s_sleep(1);
      }
      if (k >= 1) {
        const SliceStats sD = slice_stats(red_max[par][0], red_sum[par][0]);
        const SliceStats sT = slice_stats(red_max[par][1], red_sum[par][1]);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          if (lane + h * kWave == g) {  // this workgroup's own word, as the others read it
            const uint32_t tg = epoch_tag(epoch);
            ad[h] = __uint_as_float(tagged(sD.a, tg)); sd[h] = __uint_as_float(tagged(sD.s, tg));
            at[h] = __uint_as_float(tagged(sT.a, tg)); st[h] = __uint_as_float(tagged(sT.s, tg));
          }
        }
        // row normaliser in log2 units: off = M + log2(sum_j s_j 2^{a_j - M})
        const float MD = wave_max(vmax(sd[0] > 0.f ? ad[0] : -INFINITY, sd[1] > 0.f ? ad[1] : -INFINITY));
        const float MT = wave_max(vmax(st[0] > 0.f ? at[0] : -INFINITY, st[1] > 0.f ? at[1] : -INFINITY));
        float xD = 0.f, xT = 0.f;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          xD += sd[h] > 0.f ? sd[h] * exp2_fast(ad[h] - MD) : 0.f;
          xT += st[h] > 0.f ? st[h] * exp2_fast(at[h] - MT) : 0.f;
        }
        const float SD = wave_sum(xD), ST = wave_sum(xT);
        const bool poisoned = __any(!ok);
        if (lane == 0) {
          glob[par][0] = poisoned ? NAN : sD.a - (MD + __builtin_amdgcn_logf(SD));
          glob[par][1] = poisoned ? NAN : sT.a - (MT + __builtin_amdgcn_logf(ST));
        }
      }
      // after the polls, so that their wait never includes this store
      if (k >= 2) store_share(k - 2);
      __syncthreads();  // B
      if (k < nk && lane == 0) {
        const int pk = (int)(k & 1);
        const SliceStats sD = slice_stats(red_max[pk][0], red_sum[pk][0]);
        const SliceStats sT = slice_stats(red_max[pk][1], red_sum[pk][1]);
        publish(cslots + (size_t)pk * G + g, sD.a, sD.s, sT.a, sT.s, (uint32_t)k + 1u);
      }
    }
    __syncthreads();
    if (nk >= 1) store_share(nk - 1);
  }
}

// accept[row] = clamp(sum_g share[row][g], 0, 1) in fixed order, and tau per
// block of gamma rows (page 1 §3.10); one thread per block.
// One thread per row: the row's G shares in a fixed order (four independent
// partial sums, so the loads go out together; results are deterministic),
// clamped.  When gamma divides the wave width, a block's rows sit in gamma
// consecutive lanes and tau = 1 + sum_k prod_{i<=k} a_i m_i is a segmented
// prefix product and sum over them; otherwise tau_kernel runs afterwards.
__global__ void tv_finalize_kernel(const float* __restrict__ share, int G,
                                   float* __restrict__ accept, const uint8_t* __restrict__ m,
                                   float* __restrict__ tau, int64_t rows, int gamma) {
  const int64_t row = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  float a = 0.f;
  if (row < rows) {
    const float* sp = share + row * G;
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
    int j = 0;
    for (; j + 4 <= G; j += 4) {
      s0 += sp[j];
      s1 += sp[j + 1];
      s2 += sp[j + 2];
      s3 += sp[j + 3];
    }
    for (; j < G; ++j) s0 += sp[j];
    const float x = (s0 + s1) + (s2 + s3);
    a = x != x ? x : fminf(fmaxf(x, 0.f), 1.f);  // a poisoned (NaN) row stays NaN
    accept[row] = a;
  }
  if (!tau || kWave % gamma != 0) return;
  const int k = (int)(threadIdx.x % gamma);  // rows of a block are consecutive lanes
  float run = (row < rows) ? a * (m ? (float)(m[row] != 0) : 1.f) : 0.f;
  for (int off = 1; off < gamma; off <<= 1) {
    const float y = __shfl_up(run, off, kWave);
    if (k >= off) run *= y;
  }
  float sum = run;
  for (int off = gamma >> 1; off > 0; off >>= 1) sum += __shfl_xor(sum, off, kWave);
  if (k == 0 && row < rows) tau[row / gamma] = 1.f + sum;
}

__global__ void zero_u32_kernel(unsigned* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// Fallback for rows that are not 16-byte aligned (V not a multiple of the
// vector width) or too long for one cluster: one workgroup per row, three
// streaming passes over global memory.  Correctness path only.
constexpr int kRowThreads = 256;

template <bool kMax>
__device__ __forceinline__ float block_reduce(float v, float* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  v = kMax ? wave_max(v) : wave_sum(v);
  __syncthreads();  // red[] may still be read by the previous reduction
  if (lane == 0) red[w] = v;
  __syncthreads();
  return kMax ? vmax(vmax(red[0], red[1]), vmax(red[2], red[3]))
              : (red[0] + red[1]) + (red[2] + red[3]);
}

template <bool kBf16>
__global__ __launch_bounds__(kRowThreads) void tv_rowwise_kernel(const void* __restrict__ d,
                                                                 const void* __restrict__ t,
                                                                 float* __restrict__ accept,
                                                                 int64_t rows, int V) {
  __shared__ float red[4];
  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    auto ld = [&](const void* p, int v) -> float {
      if (kBf16) {
        const uint16_t h = ((const uint16_t*)p)[row * V + v];
        return __uint_as_float((uint32_t)h << 16);
      }
      return ((const float*)p)[row * V + v];
    };
    float md = -INFINITY, mt = -INFINITY;
    for (int v = threadIdx.x; v < V; v += kRowThreads) {
      md = fmaxf(md, ld(d, v));
      mt = fmaxf(mt, ld(t, v));
    }
    md = block_reduce<true>(md, red);
    mt = block_reduce<true>(mt, red);
    float sd = 0.f, st = 0.f;
    for (int v = threadIdx.x; v < V; v += kRowThreads) {
      sd += exp2_fast((ld(d, v) - md) * kLog2e);
      st += exp2_fast((ld(t, v) - mt) * kLog2e);
    }
    sd = block_reduce<false>(sd, red);
    st = block_reduce<false>(st, red);
    const float offd = md * kLog2e + __builtin_amdgcn_logf(sd);
    const float offt = mt * kLog2e + __builtin_amdgcn_logf(st);
    float s = 0.f;
    for (int v = threadIdx.x; v < V; v += kRowThreads)
      s += exp2_fast(fminf(fmaf(ld(d, v), kLog2e, -offd), fmaf(ld(t, v), kLog2e, -offt)));
    s = block_reduce<false>(s, red);
    if (threadIdx.x == 0) accept[row] = fminf(fmaxf(s, 0.f), 1.f);
  }
}

// tau[b,a] = 1 + sum_k prod_{i<=k} accept[b,a,i] * m[b,a,i]   (page 1 §3.10)
__global__ void tau_kernel(const float* __restrict__ accept, const uint8_t* __restrict__ m,
                           float* __restrict__ tau, int64_t nblocks, int gamma) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nblocks) return;
  float run = 1.f, s = 0.f;
  for (int k = 0; k < gamma; ++k) {
    const float w = accept[i * gamma + k] * (m ? (float)(m[i * gamma + k] != 0) : 1.f);
    run *= w;
    s += run;
  }
  tau[i] = 1.f + s;
}

int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  return cus;
}

// Cluster geometry: G workgroups per row, each holding kChunkVec vectors of
// each tensor (the last one fewer).  Zero G means the row-wise fallback.
struct Geometry {
  int vec_per_row, G;
};
Geometry geometry(int V, int dtype) {
  const int epv = dtype == DSPARK_BF16 ? 8 : 4;
  if (V % epv != 0) return {0, 0};
  const int vpr = V / epv;
  const int G = (vpr + kChunkVec - 1) / kChunkVec;
  return {vpr, G <= kMaxG ? G : 0};
}
// Device-independent bound on resident clusters, for the workspace size:
// at most 16 workgroups per compute unit on 256 compute units.
int64_t max_clusters(int64_t rows, int G) {
  int64_t cl = (256 * 16) / G;
  return cl < rows ? cl : rows;
}

}  // namespace

extern "C" size_t dspark_accept_rate_workspace_bytes(int B, int A, int gamma, int V, int dtype) {
  using dspark_host::align_up;
  if (B < 0 || A < 0 || gamma < 0 || V < 0) return 0;
  const int64_t rows = (int64_t)B * A * gamma;
  const Geometry geo = geometry(V, dtype);
  if (geo.G == 0 || rows == 0) return 0;
  const size_t shares = align_up((size_t)rows * geo.G * sizeof(float), 256);
  const size_t slots = (size_t)max_clusters(rows, geo.G) * 2 * geo.G * sizeof(u32x4);
  return shares + slots + 64;
}

// Poll limit of the cooperative waits; 0 selects kSpinLimit.
static std::atomic<uint32_t> g_wait_limit{0};

extern "C" void dspark_set_wait_limit(uint32_t polls) {
  g_wait_limit.store(polls, std::memory_order_relaxed);
}

namespace dspark {
uint32_t wait_limit() {
  const uint32_t lim = g_wait_limit.load(std::memory_order_relaxed);
  return lim ? lim : kSpinLimit;
}
}  // namespace dspark

extern "C" int dspark_accept_rate(const void* draft_logits, const void* target_logits,
                                  float* accept, const uint8_t* eval_mask, float* tau, int B,
                                  int A, int gamma, int V, int dtype, void* ws, size_t ws_bytes,
                                  int32_t* dev_status, void* stream) {
  using namespace dspark_host;
  if (B < 0 || A < 0 || gamma < 0)
    return fail(DSPARK_ERR_INVALID_ARG, "accept_rate: negative dimension");
  if (dtype != DSPARK_BF16 && dtype != DSPARK_F32)
    return fail(DSPARK_ERR_INVALID_ARG, "accept_rate: unknown dtype %d", dtype);
  if (V < 2) return fail(DSPARK_ERR_INVALID_ARG, "accept_rate: V must be >= 2 (got %d)", V);
  if (gamma > 1024) return fail(DSPARK_ERR_INVALID_ARG, "accept_rate: gamma > 1024");
  const int64_t rows = (int64_t)B * A * gamma;
  if (rows == 0) return ok();
  if (!draft_logits || !target_logits || !accept)
    return fail(DSPARK_ERR_INVALID_ARG, "accept_rate: null required pointer");
  const size_t need = dspark_accept_rate_workspace_bytes(B, A, gamma, V, dtype);
  if (ws_bytes < need || (need > 0 && !ws))
    return fail(DSPARK_ERR_WORKSPACE, "accept_rate: workspace %zu bytes < %zu", ws_bytes, need);
  hipStream_t s = (hipStream_t)stream;
  const bool bf = dtype == DSPARK_BF16;
  const bool aligned = ((uintptr_t)draft_logits % 16 == 0) && ((uintptr_t)target_logits % 16 == 0);
  const Geometry geo = geometry(V, dtype);
  const void* kern = bf ? (const void*)tv_cluster_kernel<true> : (const void*)tv_cluster_kernel<false>;
  int64_t ncl = 0;
  if (geo.G > 0 && aligned) {
    const int cap = cluster_capacity(kern, kThreads, "accept_rate");
    if (cap <= 0) return fail(DSPARK_ERR_HIP, "accept_rate: occupancy query failed");
    ncl = cap / geo.G;
    const int64_t bound = max_clusters(rows, geo.G);
    if (ncl > bound) ncl = bound;
  }
  const int64_t nb = (int64_t)B * A;
  if (ncl >= 1) {
    float* share = (float*)ws;
    u32x4* slots = (u32x4*)((char*)ws + align_up((size_t)rows * geo.G * sizeof(float), 256));
    const int64_t nslot = ncl * 2 * geo.G;
    // timeouts go to the caller's status word, else to a spare word after the slots
    int32_t* err = dev_status ? dev_status : (int32_t*)(slots + nslot);
    // slots (epoch 0 = empty) and the error word start at zero: a fill
    // kernel, not a memset node, so the sequence stays safe under graph capture
    const int64_t nwords = nslot * 4 + 1;
    hipLaunchKernelGGL(zero_u32_kernel, dim3((unsigned)((nwords + 255) / 256)), dim3(256), 0, s,
                       (unsigned*)slots, (int)nwords);
    const char* dp = (const char*)draft_logits;
    const char* tp = (const char*)target_logits;
    int64_t rows_arg = rows;
    int Varg = V, vpr = geo.vec_per_row, G = geo.G, ncl_arg = (int)ncl;
    const uint32_t lim = g_wait_limit.load(std::memory_order_relaxed);
    unsigned spin = lim ? lim : kSpinLimit;
    void* args[] = {(void*)&dp, (void*)&tp, (void*)&share, (void*)&rows_arg, (void*)&Varg,
                    (void*)&vpr, (void*)&G, (void*)&ncl_arg, (void*)&slots, (void*)&err,
                    (void*)&spin};
    if (getenv("DSPARK_VERBOSE"))
      fprintf(stderr, "[dspark] accept_rate: %d CUs, G=%d, clusters=%lld, vec/row=%d\n",
              device_cus(), G, (long long)ncl, vpr);
    hipError_t e = hipLaunchCooperativeKernel(kern, dim3((unsigned)(ncl * G)), dim3(kThreads),
                                              args, 0, s);
    if (e != hipSuccess)
      return fail(DSPARK_ERR_HIP, "accept_rate: cooperative launch: %s", hipGetErrorString(e));
    hipLaunchKernelGGL(tv_finalize_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s,
                       (const float*)share, G, accept, eval_mask, tau, rows, gamma);
    if (tau && kWave % gamma != 0)
      hipLaunchKernelGGL(tau_kernel, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, s, accept,
                         eval_mask, tau, nb, gamma);
  } else {
    int64_t grid = rows < 65536 ? rows : 65536;
    if (bf)
      hipLaunchKernelGGL(tv_rowwise_kernel<true>, dim3((unsigned)grid), dim3(kRowThreads), 0, s,
                         draft_logits, target_logits, accept, rows, V);
    else
      hipLaunchKernelGGL(tv_rowwise_kernel<false>, dim3((unsigned)grid), dim3(kRowThreads), 0, s,
                         draft_logits, target_logits, accept, rows, V);
    if (tau)
      hipLaunchKernelGGL(tau_kernel, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, s, accept,
                         eval_mask, tau, nb, gamma);
  }
  return check_launch("accept_rate");
}
