// L1 (total-variation) alignment loss of the draft logits against the target
// logits, its gradient with respect to the draft logits, and tau_greedy
// (page 1, "03 · DSpark 建模", §3.9 the paper's Eq. 10 and §3.10; page 4,
// "DSpark 深度解读", §4.1).
//
// For row n (block position k of block (b, a)) with p = softmax(draft),
// q = softmax(target):
//
//   l1_n   = sum_v |p_v - q_v|                       (twice the TV distance)
//   c_n    = w_k m_n / sum_n' w_k' m_n',  w_k = exp(-k / decay)
//   loss   = sum_n c_n l1_n
//   grad_n = c_n p_v (s_v - sum_u s_u p_u),  s = sign(p - q)
//   greedy_n = [argmax draft_n == argmax target_n]  (lowest index on ties)
//   tau_greedy[b, a] = 1 + sum_k prod_{i <= k} greedy_i m_i
//
// Two gfx950 paths, both with every reduction in a fixed order (deterministic
// results):
// * Rows of 16-byte vectors (V a multiple of 8 for bf16, of 4 for float32,
//   aligned buffers, V up to 128 x 3072): the cluster kernel below reads each
//   logit from HBM once and writes each gradient element once.
// * Otherwise one 16-wave workgroup per row and one workgroup per compute
//   unit: pass one takes each thread's online (max, sum of exponentials) and
//   argmax in one sweep, pass two the row's L1 distance and sum_u s_u p_u,
//   and pass three (only when the gradient is wanted) writes c p (s - S),
//   each pass reading the row again.
#include <limits.h>
#include <stdlib.h>

#include <algorithm>

#include "cluster.h"
#include "common.h"

using namespace dspark;

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// Running (max, sum of 2^{(x - max) log2e}, index of the first maximum).
struct Soft {
  float m, s;
  int i;
};
__device__ __forceinline__ void soft_add(Soft& a, float x, int idx) {
  if (x > a.m) {
    a.s = (a.m == -INFINITY ? 0.f : a.s * ex2((a.m - x) * kLog2e)) + 1.f;
    a.m = x;
    a.i = idx;
  } else if (x != -INFINITY) {
    a.s += ex2((x - a.m) * kLog2e);
  }
}
__device__ __forceinline__ Soft soft_merge(Soft a, Soft b) {
  if (b.m > a.m || (b.m == a.m && b.i < a.i)) { const Soft t = a; a = b; b = t; }  // a holds the winner
  if (b.m != -INFINITY) a.s += b.s * ex2((b.m - a.m) * kLog2e);
  return a;
}
__device__ __forceinline__ Soft soft_shfl(const Soft& a, int mask) {
  return Soft{__shfl_xor(a.m, mask, kWave), __shfl_xor(a.s, mask, kWave), __shfl_xor(a.i, mask, kWave)};
}

template <int N>
__device__ __forceinline__ void block_sum(float (&v)[N], float (*red)[kWaves]) {
#pragma unroll
  for (int j = 0; j < N; ++j)
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v[j] += __shfl_xor(v[j], off, kWave);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __syncthreads();  // red may still be read by the previous reduction
  if (lane == 0)
#pragma unroll
    for (int j = 0; j < N; ++j) red[j][w] = v[j];
  __syncthreads();
#pragma unroll
  for (int j = 0; j < N; ++j) {
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < kWaves; ++k) t += red[j][k];
    v[j] = t;
  }
}

template <bool kBf16>
__device__ __forceinline__ float load_elem(const void* p, int64_t i) {
  return kBf16 ? __uint_as_float((uint32_t)((const uint16_t*)p)[i] << 16) : ((const float*)p)[i];
}

// Visit the elements of a row: 16-byte vectors (8 bf16 or 4 fp32 values) when
// VEC, else one element at a time; f(value_d, value_t, index).
template <bool kBf16, bool VEC, class F>
__device__ __forceinline__ void for_row(const void* d, const void* t, int64_t row, int V, F&& f) {
  const int64_t base = row * (int64_t)V;
  if constexpr (VEC) {
    constexpr int kEl = kBf16 ? 8 : 4;
    const int nv = V / kEl;
    const char* dp = (const char*)d + base * (kBf16 ? 2 : 4);
    const char* tp = (const char*)t + base * (kBf16 ? 2 : 4);
    for (int c = threadIdx.x; c < nv; c += kThreads) {
      const u32x4 a = ((const u32x4*)dp)[c], b = ((const u32x4*)tp)[c];
#pragma unroll
      for (int e = 0; e < kEl; ++e) {
        const float x = kBf16 ? ((e & 1) ? bf16hi(a[e / 2]) : bf16lo(a[e / 2])) : __uint_as_float(a[e]);
        const float y = kBf16 ? ((e & 1) ? bf16hi(b[e / 2]) : bf16lo(b[e / 2])) : __uint_as_float(b[e]);
        f(x, y, c * kEl + e);
      }
    }
  } else {
    for (int v = threadIdx.x; v < V; v += kThreads) f(load_elem<kBf16>(d, base + v), load_elem<kBf16>(t, base + v), v);
  }
}

template <bool kBf16, bool VEC>
__global__ __launch_bounds__(kThreads) void l1_rows_kernel(const void* __restrict__ d, const void* __restrict__ t,
                                                           const float* __restrict__ coef, float* __restrict__ row_l1,
                                                           float* __restrict__ greedy, float* __restrict__ grad,
                                                           int64_t rows, int V) {
  __shared__ float red[3][kWaves];
  __shared__ Soft sred[2][kWaves];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    // pass one: online softmax statistics and argmax of both rows
    Soft sd{-INFINITY, 0.f, INT_MAX}, st{-INFINITY, 0.f, INT_MAX};
    for_row<kBf16, VEC>(d, t, row, V, [&](float x, float y, int v) {
      soft_add(sd, x, v);
      soft_add(st, y, v);
    });
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      sd = soft_merge(sd, soft_shfl(sd, off));
      st = soft_merge(st, soft_shfl(st, off));
    }
    __syncthreads();  // sred may still be read for the previous row
    if (lane == 0) { sred[0][w] = sd; sred[1][w] = st; }
    __syncthreads();
    sd = sred[0][0];
    st = sred[1][0];
#pragma unroll
    for (int k = 1; k < kWaves; ++k) {
      sd = soft_merge(sd, sred[0][k]);
      st = soft_merge(st, sred[1][k]);
    }
    // p_v = 2^{(x - m) log2e} / s; a row of -inf logits has no distribution
    const float md = sd.m == -INFINITY ? 0.f : sd.m * kLog2e, id = 1.f / sd.s;
    const float mt = st.m == -INFINITY ? 0.f : st.m * kLog2e, it = 1.f / st.s;
    // pass two: l1 = sum |p - q| and S = sum sign(p - q) p
    float acc[2] = {0.f, 0.f};
    for_row<kBf16, VEC>(d, t, row, V, [&](float x, float y, int) {
      // both distributions rounded the same way before they meet (a fused
      // p - e * it would make identical rows differ)
#pragma clang fp contract(off)
      const float p = ex2(fmaf(x, kLog2e, -md)) * id, q = ex2(fmaf(y, kLog2e, -mt)) * it;
      const float dlt = p - q;
      acc[0] += fabsf(dlt);
      acc[1] += dlt > 0.f ? p : (dlt < 0.f ? -p : 0.f);
    });
    block_sum(acc, red);
    if (threadIdx.x == 0) {
      if (row_l1) row_l1[row] = acc[0];
      greedy[row] = sd.i == st.i ? 1.f : 0.f;
    }
    if (grad) {
      // pass three: grad = c p (s - S)
      const float cf = coef[row], S = acc[1];
      float* g = grad + row * (int64_t)V;
      for_row<kBf16, VEC>(d, t, row, V, [&](float x, float y, int v) {
#pragma clang fp contract(off)
        const float p = ex2(fmaf(x, kLog2e, -md)) * id, q = ex2(fmaf(y, kLog2e, -mt)) * it;
        const float sg = p > q ? 1.f : (p < q ? -1.f : 0.f);
        g[v] = cf * p * (sg - S);
      });
    }
  }
}

// ---------------------------------------------------------------- cluster path
// HBM-bound design: a row (2 x V logits) is split over a cluster of G
// co-resident workgroups (cooperative grid), each holding a 3072-element slice
// of both tensors in registers and LDS, so every logit is read from HBM once
// and the gradient written once.  Three data waves do the arithmetic; an
// exchange wave trades each row's per-slice statistics with the cluster
// through global memory twice: the softmax statistics (max, sum of
// exponentials relative to the slice maximum) after pass one, and the slice's
// share of S = sum_v s_v p_v after pass two, which the gradient needs.  The
// row passes are pipelined over the cluster's rows so that each exchange has a
// whole iteration to complete: iteration k runs pass one of row k (max, first
// index of the maximum, exponentials and their sums, parked in LDS), pass two
// of row k-1 (p, q, the slice's sum |p - q| and sum s p; p kept in LDS with
// the sign of p - q) and pass three of row k-3 (c p (s - S), written out).
// Each workgroup writes its slice's L1 share and maxima to a record; a small
// kernel folds the G records of a row in fixed order (deterministic).
constexpr int kCDataWaves = 3;
constexpr int kCDataThreads = kCDataWaves * kWave;
constexpr int kCThreads = kCDataThreads + kWave;  // plus the exchange wave
constexpr int kCN = 16;                           // elements of each tensor per data thread
constexpr int kChunkEl = kCDataThreads * kCN;     // slice length, both dtypes
constexpr int kCMaxG = 2 * kWave;                 // two cluster members per exchange lane
constexpr uint32_t kSCopies = 4;                  // rotating slots of the S exchange
static_assert(kChunkEl < 65536, "slice indices are packed as 16-bit fields");

template <bool kBf16>
struct CShape {
  static constexpr int kEl = kBf16 ? 8 : 4;                // elements per 16-byte vector
  static constexpr int kVec = kCN / kEl;                   // vectors per tensor per data thread
  static constexpr int kChunkVec = kCDataThreads * kVec;   // vectors per tensor per workgroup
};

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, off, kWave));
  return v;
}

// p (>= 0) of pass two with the sign of p - q in the sign bit and a tie flag
// (p == q) in the lowest mantissa bit, which is dropped from p: the gradient
// uses p to within one unit in its last place.
__device__ __forceinline__ uint32_t encode_p(float p, float dl) {
  return (__float_as_uint(p) & 0x7ffffffeu) | (__float_as_uint(dl) & 0x80000000u) | (dl == 0.f ? 1u : 0u);
}

// Workspace records rec[row][g]: {slice L1 share, slice max of draft, slice
// max of target, (first index of the draft max << 16) | first index of the
// target max}, indices relative to the slice start.
template <bool kBf16, bool kGrad>
__global__ __launch_bounds__(kCThreads) void l1_cluster_kernel(
    const char* __restrict__ d, const char* __restrict__ t, const float* __restrict__ coef,
    float* __restrict__ grad, u32x4* __restrict__ rec, int64_t rows, int V, int vec_per_row, int G,
    int nclusters, u32x4* __restrict__ slots, uint32_t* __restrict__ sslots, int32_t* __restrict__ err,
    unsigned spin_limit) {
  using namespace dspark::cluster;
  constexpr int kEl = CShape<kBf16>::kEl, kVec = CShape<kBf16>::kVec, kQ = kCN / 4;
  __shared__ f32x4 park[2 * kQ][kCDataThreads];                          // exponentials of the next pass two
  __shared__ u32x4 cpt[kGrad ? 2 : 1][kGrad ? kQ : 1][kCDataThreads];     // encoded p by row parity
  __shared__ float red_max[2][2][kCDataWaves], red_sum[2][2][kCDataWaves];
  __shared__ uint32_t red_idx[2][2][kCDataWaves];
  __shared__ float red_part[2][kCDataWaves];  // [L1, S][wave] of the last pass two
  __shared__ float glob[2][2];                // [row parity][draft, target] exponent offsets
  __shared__ float glob_s[2];                 // S by row parity
  const int cl = blockIdx.x / G, g = blockIdx.x % G;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform role
  const uint32_t row_bytes = (uint32_t)V * (kBf16 ? 2u : 4u);
  u32x4* cslots = slots + (size_t)cl * 2 * G;
  uint32_t* csslots = sslots + (size_t)cl * kSCopies * G;
  const int64_t nk = (rows - cl + nclusters - 1) / nclusters;  // rows of this cluster (cl < rows)
  const int64_t kend = kGrad ? nk + 2 : nk + 1;                 // the last iteration drains the pipeline

  if (w < kCDataWaves) {
    // ------------------------------------------------------------ data waves
    // Global accesses of these waves: the streaming loads, and the gradient
    // stores of pass three, issued early in an iteration (right after barrier
    // A): a wave's wait for its loads also waits for every earlier store
    // (loads and stores may complete out of order, so the counter wait
    // cannot skip stores), and stores issued there have most of an iteration
    // to complete before the next wait.
    const int tid = threadIdx.x;
    const int vbase = g * CShape<kBf16>::kChunkVec;
    const uint32_t voff = (uint32_t)(vbase + tid) * 16u;
    bool full[kVec];
#pragma unroll
    for (int i = 0; i < kVec; ++i) full[i] = vbase + (i + 1) * kCDataThreads <= vec_per_row;  // uniform
    u32x4 rd[kVec], rt[kVec];
    auto issue = [&](int64_t row) {
      const bool in = row < rows;
      const int64_t off = (in ? row : 0) * (int64_t)row_bytes;
      const int nrec = in ? (int)row_bytes : 0;
      const __amdgpu_buffer_rsrc_t sd = __builtin_amdgcn_make_buffer_rsrc((void*)(d + off), 0, nrec, kRsrcWord3);
      const __amdgpu_buffer_rsrc_t st = __builtin_amdgcn_make_buffer_rsrc((void*)(t + off), 0, nrec, kRsrcWord3);
#pragma unroll
      for (int i = 0; i < kVec; ++i) {
        rd[i] = __builtin_amdgcn_raw_buffer_load_b128(sd, voff, i * kCDataThreads * 16, kNonTemporal);
        rt[i] = __builtin_amdgcn_raw_buffer_load_b128(st, voff, i * kCDataThreads * 16, kNonTemporal);
      }
    };
    // element j of this thread sits at slice offset (j / kEl * kCDataThreads + tid) * kEl + j % kEl
    auto local_index = [&](int j) { return (uint32_t)(((j / kEl) * kCDataThreads + tid) * kEl + j % kEl); };
    issue(cl);
    for (int64_t k = 0; k <= kend; ++k) {
      const int64_t row = cl + k * nclusters;
      const int par = (int)(k & 1);
      float xd[kCN], xt[kCN];
      float tmd = -INFINITY, tmt = -INFINITY;
      if (k < nk) {
#pragma unroll
        for (int i = 0; i < kVec; ++i) {
          const bool valid = full[i] || vbase + i * kCDataThreads + tid < vec_per_row;
          const uint32_t pad = valid ? 0u : 0xff800000u;  // past the row end: -inf
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            if (kBf16) {
              xd[i * 8 + 2 * c] = __uint_as_float((rd[i][c] << 16) | pad);
              xd[i * 8 + 2 * c + 1] = __uint_as_float((rd[i][c] & 0xffff0000u) | pad);
              xt[i * 8 + 2 * c] = __uint_as_float((rt[i][c] << 16) | pad);
              xt[i * 8 + 2 * c + 1] = __uint_as_float((rt[i][c] & 0xffff0000u) | pad);
            } else {
              xd[i * 4 + c] = __uint_as_float(rd[i][c] | pad);
              xt[i * 4 + c] = __uint_as_float(rt[i][c] | pad);
            }
          }
        }
        issue(row + nclusters);  // the next row streams in while this one is reduced
#pragma unroll
        for (int j = 0; j < kCN; ++j) {
          tmd = vmax(tmd, xd[j]);
          tmt = vmax(tmt, xt[j]);
        }
        const float md = wave_max(tmd), mt = wave_max(tmt);
        if (lane == 0) { red_max[par][0][w] = md; red_max[par][1][w] = mt; }
      }
      __syncthreads();  // A: slice maxima of row k; S of row k-3 is in LDS
      if (kGrad && k >= 3 && k - 3 < nk) {
        // pass three of row k-3: grad = c p (s - S) on the encoded p
        const int64_t r3 = row - 3 * nclusters;
        const int p3 = (int)((k - 3) & 1);
        const float S = uniform(glob_s[p3]);
        const float cf = coef[r3];
        const float cA = cf * (1.f - S), cB = cf * (-1.f - S), cC = cf * (-S);
        float* gp = grad + r3 * (int64_t)V + (int64_t)vbase * kEl;
#pragma unroll
        for (int i = 0; i < kVec; ++i) {
          float o[kEl];
#pragma unroll
          for (int e = 0; e < kEl; ++e) {
            const int j = i * kEl + e;
            const uint32_t wv = cpt[p3][j / 4][tid][j % 4];
            const float f = (wv & 1u) ? cC : ((int32_t)wv < 0 ? cB : cA);
            o[e] = __uint_as_float(wv & 0x7ffffffeu) * f;
          }
          if (full[i] || vbase + i * kCDataThreads + tid < vec_per_row) {
            f32x4* dst = (f32x4*)(gp + (int64_t)(i * kCDataThreads + tid) * kEl);
#pragma unroll
            for (int h = 0; h < kEl / 4; ++h) dst[h] = f32x4{o[4 * h], o[4 * h + 1], o[4 * h + 2], o[4 * h + 3]};
          }
        }
      }
      if (k < nk) {
        const float mD = vmax(vmax(red_max[par][0][0], red_max[par][0][1]), red_max[par][0][2]);
        const float mT = vmax(vmax(red_max[par][1][0], red_max[par][1][1]), red_max[par][1][2]);
        // first index of the slice maximum: only lanes that hold it search
        uint32_t cd = 0xffffffffu, ct = 0xffffffffu;
        if (tmd == mD) {
#pragma unroll
          for (int j = kCN - 1; j >= 0; --j) cd = xd[j] == mD ? local_index(j) : cd;
        }
        if (tmt == mT) {
#pragma unroll
          for (int j = kCN - 1; j >= 0; --j) ct = xt[j] == mT ? local_index(j) : ct;
        }
        cd = wave_min_u32(cd);
        ct = wave_min_u32(ct);
        const float aD = mD == -INFINITY ? 0.f : mD * kLog2e;
        const float aT = mT == -INFINITY ? 0.f : mT * kLog2e;
        float sd0 = 0.f, sd1 = 0.f, st0 = 0.f, st1 = 0.f;
#pragma unroll
        for (int j = 0; j < kCN; j += 2) {
          xd[j] = exp2_fast(fmaf(xd[j], kLog2e, -aD));
          xd[j + 1] = exp2_fast(fmaf(xd[j + 1], kLog2e, -aD));
          xt[j] = exp2_fast(fmaf(xt[j], kLog2e, -aT));
          xt[j + 1] = exp2_fast(fmaf(xt[j + 1], kLog2e, -aT));
          sd0 += xd[j]; sd1 += xd[j + 1];
          st0 += xt[j]; st1 += xt[j + 1];
        }
        const float wsd = wave_sum(sd0 + sd1), wst = wave_sum(st0 + st1);
        if (lane == 0) {
          red_sum[par][0][w] = wsd; red_sum[par][1][w] = wst;
          red_idx[par][0][w] = cd; red_idx[par][1][w] = ct;
        }
      }
      __syncthreads();  // B: sums of row k; offsets of row k-1 are in LDS
      if (k >= 1 && k - 1 < nk) {
        // pass two of row k-1 on its parked exponentials: p = e_d 2^{eD}, q = e_t 2^{eT}
        const int p1 = (int)((k - 1) & 1);
        const float scD = exp2_fast(uniform(glob[p1][0])), scT = exp2_fast(uniform(glob[p1][1]));
        float l0 = 0.f, l1 = 0.f, s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int q4 = 0; q4 < kQ; ++q4) {
          const f32x4 a = park[q4][tid], b = park[kQ + q4][tid];
          u32x4 enc;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            // both distributions rounded the same way before they meet (a
            // fused p - e_t 2^{eT} would make identical rows differ)
#pragma clang fp contract(off)
            const float p = a[e] * scD, q = b[e] * scT;
            const float dl = p - q;
            const float sp = dl > 0.f ? p : (dl < 0.f ? -p : 0.f);
            if (e & 1) { l1 += fabsf(dl); s1 += sp; } else { l0 += fabsf(dl); s0 += sp; }
            enc[e] = encode_p(p, dl);
          }
          if (kGrad) cpt[p1][q4][tid] = enc;  // the slot of row k-3, read above
        }
        const float wl = wave_sum(l0 + l1), ws = wave_sum(s0 + s1);
        if (lane == 0) { red_part[0][w] = wl; red_part[1][w] = ws; }
      }
      if (k < nk) {
#pragma unroll
        for (int q4 = 0; q4 < kQ; ++q4) {
          park[q4][tid] = f32x4{xd[4 * q4], xd[4 * q4 + 1], xd[4 * q4 + 2], xd[4 * q4 + 3]};
          park[kQ + q4][tid] = f32x4{xt[4 * q4], xt[4 * q4 + 1], xt[4 * q4 + 2], xt[4 * q4 + 3]};
        }
      }
    }
  } else {
    // --------------------------------------------------------- exchange wave
    // It also does every global store of the workgroup other than the
    // gradient (published words, records), and issues ahead of the data
    // waves on its SIMD: its short, latency-bound sequence decides when they
    // may pass the barriers.  Per iteration k: at A, the L1 share and the S
    // share of row k-2 (pass two ran in iteration k-1); before B, the
    // cluster's statistics of row k-1 (published after their B of iteration
    // k-1); after B, this slice's statistics of row k, then the cluster's S
    // shares of row k-2 (published at their A of iteration k), needed by pass
    // three after A of iteration k+1.  Each gather has an iteration to
    // complete, so the members drift by at most one iteration.
    __builtin_amdgcn_s_setprio(3);
    bool ok = true;       // after one timed-out wait this lane stops waiting
    // Wait until every lane holds its members' words; give up on a member
    // after the poll bound (the row is poisoned).
    auto gather = [&](bool* got, auto&& try_fetch) {
      unsigned n = 0;
      while (!__all(got[0] && got[1])) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          if (!got[h]) {
            if (try_fetch(h)) {
              got[h] = true;
            } else if (!ok || ++n > spin_limit) {
              if (ok) atomicOr(err, DSPARK_STATUS_WAIT_TIMEOUT);
              ok = false;
              got[h] = true;
            }
          }
        }
        if (!__all(got[0] && got[1])) __builtin_amdgcn_s_sleep(1);
      }
    };
    for (int64_t k = 0; k <= kend; ++k) {
      const int64_t row = cl + k * nclusters;
      const bool have2 = k >= 2 && k - 2 < nk;  // row k-2 finished pass two
      uint32_t word2 = 0;                       // this member's tagged S word of row k-2
      __syncthreads();  // A
      if (have2) {
        const float l1g = (red_part[0][0] + red_part[0][1]) + red_part[0][2];
        const float sg = (red_part[1][0] + red_part[1][1]) + red_part[1][2];
        word2 = tagged(sg, epoch_tag_n((uint32_t)(k - 2), kSCopies));
        if (lane == 0) {
          ((float*)(rec + (row - 2 * nclusters) * G + g))[0] = l1g;
          if (kGrad) publish32(csslots + (size_t)((k - 2) & (kSCopies - 1)) * G + g, word2);
        }
      }
      if (k >= 1 && k - 1 < nk) {
        // statistics of row k-1 (published as epoch k)
        const int par = (int)((k - 1) & 1);
        const uint32_t epoch = (uint32_t)k;
        float ad[2] = {-INFINITY, -INFINITY}, sd[2] = {0.f, 0.f};
        float at[2] = {-INFINITY, -INFINITY}, st[2] = {0.f, 0.f};
        bool got[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int j = lane + h * kWave;
          got[h] = j >= G || j == g;  // nothing to fetch
        }
        gather(got, [&](int h) {
          const u32x4 v = peek(cslots + (size_t)par * G + lane + h * kWave);
          if (!fresh(v, epoch)) return false;
          ad[h] = __uint_as_float(v[0]); sd[h] = __uint_as_float(v[1]);
          at[h] = __uint_as_float(v[2]); st[h] = __uint_as_float(v[3]);
          return true;
        });
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
      __syncthreads();  // B
      if (k < nk && lane == 0) {
        const int pk = (int)(k & 1);
        const SliceStats sD = slice_stats(red_max[pk][0], red_sum[pk][0]);
        const SliceStats sT = slice_stats(red_max[pk][1], red_sum[pk][1]);
        publish(cslots + (size_t)pk * G + g, sD.a, sD.s, sT.a, sT.s, (uint32_t)k + 1u);
        const float mD = vmax(vmax(red_max[pk][0][0], red_max[pk][0][1]), red_max[pk][0][2]);
        const float mT = vmax(vmax(red_max[pk][1][0], red_max[pk][1][1]), red_max[pk][1][2]);
        const uint32_t iD = min(min(red_idx[pk][0][0], red_idx[pk][0][1]), red_idx[pk][0][2]);
        const uint32_t iT = min(min(red_idx[pk][1][0], red_idx[pk][1][1]), red_idx[pk][1][2]);
        uint32_t* r = (uint32_t*)(rec + row * G + g);
        r[1] = __float_as_uint(mD);
        r[2] = __float_as_uint(mT);
        r[3] = (iD << 16) | (iT & 0xffffu);
      }
      if (kGrad && have2) {
        // S of row k-2: the same words in the same order on every member
        const uint32_t tag2 = epoch_tag_n((uint32_t)(k - 2), kSCopies);
        const uint32_t* s2 = csslots + (size_t)((k - 2) & (kSCopies - 1)) * G;
        float sv[2] = {0.f, 0.f};
        bool got[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int j = lane + h * kWave;
          got[h] = j >= G;
          if (j == g) { sv[h] = __uint_as_float(word2); got[h] = true; }
        }
        gather(got, [&](int h) {
          const uint32_t v = peek32(s2 + lane + h * kWave);
          if ((v & 1u) != tag2) return false;
          sv[h] = __uint_as_float(v);
          return true;
        });
        const float S = wave_sum(sv[0] + sv[1]);
        const bool poisoned = __any(!ok);
        if (lane == 0) glob_s[(k - 2) & 1] = poisoned ? NAN : S;
      }
    }
  }
}

// Per row: L1 = sum of the G slice shares (a fixed reduction tree) and the
// greedy flag from the first maxima (slices in index order, so the first
// slice that holds the row maximum holds its lowest index).  One wave per
// row: lane g reads slice records g and g + 64 (consecutive 16-byte records,
// coalesced), then the wave folds sums and (maximum, lowest slice) keys.
__device__ __forceinline__ uint64_t first_max_key(float v, int g) {
  return ((uint64_t)float_order_key(v) << 32) | (uint64_t)(0xffffffffu - (uint32_t)g);
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t k) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)k, off, kWave), hi = __shfl_xor((uint32_t)(k >> 32), off, kWave);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    k = o > k ? o : k;
  }
  return k;
}
constexpr int kFinRows = 4;  // rows (waves) per workgroup
__global__ __launch_bounds__(64 * kFinRows) void l1_cluster_finalize_kernel(const u32x4* __restrict__ rec, int G,
                                                                          float* __restrict__ row_l1,
                                                                          float* __restrict__ greedy, int64_t rows) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kFinRows + (threadIdx.x >> 6);
  if (row >= rows) return;  // whole waves
  const u32x4* r = rec + row * G;
  float l = 0.f;
  uint64_t kd = 0, kt = 0;  // 0: no slice (below every real key)
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int g = lane + 64 * h;
    if (g < G) {
      const u32x4 x = r[g];
      l += __uint_as_float(x[0]);
      const uint64_t d = first_max_key(__uint_as_float(x[1]), g), t = first_max_key(__uint_as_float(x[2]), g);
      kd = d > kd ? d : kd;
      kt = t > kt ? t : kt;
    }
  }
  l = cluster::wave_sum(l);
  kd = wave_max_u64(kd);
  kt = wave_max_u64(kt);
  // the winning slices' first-maximum positions
  const int gd = (int)(0xffffffffu - (uint32_t)kd), gt = (int)(0xffffffffu - (uint32_t)kt);
  const uint32_t pd = rec[row * G + gd][3] >> 16, pt = rec[row * G + gt][3] & 0xffffu;
  if (lane == 0) {
    row_l1[row] = l;
    greedy[row] = (uint32_t)gd * kChunkEl + pd == (uint32_t)gt * kChunkEl + pt ? 1.f : 0.f;
  }
}

__global__ void l1_zero_u32_kernel(uint32_t* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// c[n] = w_k m_n / sum(w m) with w_k = exp(-k / decay); one workgroup, fixed
// summation order.  All zeros when no position is valid.
__global__ __launch_bounds__(kThreads) void l1_coef_kernel(const uint8_t* __restrict__ m, float* __restrict__ coef,
                                                           int64_t rows, int gamma, float decay) {
  __shared__ float red[1][kWaves];
  // the position k = n mod gamma advances by kThreads mod gamma per step (no 64-bit division)
  const int step = kThreads % gamma;
  float part[1] = {0.f};
  int k = (int)threadIdx.x % gamma;
  for (int64_t n = threadIdx.x; n < rows; n += kThreads) {
    if (!m || m[n]) part[0] += expf(-(float)k / decay);
    k += step;
    if (k >= gamma) k -= gamma;
  }
  block_sum(part, red);
  const float inv = part[0] > 0.f ? 1.f / part[0] : 0.f;
  k = (int)threadIdx.x % gamma;
  for (int64_t n = threadIdx.x; n < rows; n += kThreads) {
    coef[n] = (!m || m[n]) ? expf(-(float)k / decay) * inv : 0.f;
    k += step;
    if (k >= gamma) k -= gamma;
  }
}

// loss = sum_n c_n l1_n (one workgroup, fixed order); tau_greedy per block.
__global__ __launch_bounds__(kThreads) void l1_finalize_kernel(const float* __restrict__ coef,
                                                               const float* __restrict__ row_l1,
                                                               const float* __restrict__ greedy,
                                                               const uint8_t* __restrict__ m, float* __restrict__ loss,
                                                               float* __restrict__ tau, int64_t rows, int gamma) {
  __shared__ float red[1][kWaves];
  float part[1] = {0.f};
  for (int64_t n = threadIdx.x; n < rows; n += kThreads) part[0] += coef[n] * row_l1[n];
  block_sum(part, red);
  if (threadIdx.x == 0) loss[0] = part[0];
  if (!tau) return;
  for (int64_t blk = threadIdx.x; blk < rows / gamma; blk += kThreads) {
    float run = 1.f, sum = 1.f;
    for (int k = 0; k < gamma; ++k) {
      const int64_t n = blk * gamma + k;
      run *= greedy[n] * ((!m || m[n]) ? 1.f : 0.f);
      sum += run;
    }
    tau[blk] = sum;
  }
}

int device_cu_count() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  return cus;
}

// Cluster geometry: G workgroups per row, each holding kChunkEl elements of
// each tensor (the last one fewer).  Zero G means the row-wise kernel.
struct Geometry {
  int vec_per_row, G;
};
Geometry geometry(int V, int dtype) {
  const int epv = dtype == DSPARK_BF16 ? 8 : 4;
  if (V % epv != 0) return {0, 0};
  const int G = (V + kChunkEl - 1) / kChunkEl;
  return {V / epv, G <= kCMaxG ? G : 0};
}
// Device-independent bound on resident clusters, for the workspace size:
// at most 16 workgroups per compute unit on 256 compute units.
int64_t max_clusters(int64_t rows, int G) {
  const int64_t cl = (256 * 16) / G;
  return cl < rows ? cl : rows;
}
struct Layout {
  size_t coef, l1, greedy, rec, slots, sslots, err, total;
};
Layout layout(int64_t rows, const Geometry& geo) {
  using dspark_host::align_up;
  const size_t slab = align_up((size_t)rows * sizeof(float), 256);
  Layout L{};
  L.coef = 0;
  L.l1 = slab;
  L.greedy = 2 * slab;
  L.total = 3 * slab;
  if (geo.G > 0) {
    const int64_t ncl = max_clusters(rows, geo.G);
    L.rec = L.total;
    L.slots = L.rec + align_up((size_t)rows * geo.G * sizeof(u32x4), 256);
    L.sslots = L.slots + align_up((size_t)ncl * 2 * geo.G * sizeof(u32x4), 256);
    L.err = L.sslots + align_up((size_t)ncl * kSCopies * geo.G * sizeof(uint32_t), 256);
    L.total = L.err + 256;
  }
  return L;
}

}  // namespace

// Workspace: c [rows] | l1 [rows] | greedy [rows] float32, and for rows that
// the cluster kernel takes: records [rows][G] | statistics slots | S slots |
// error word; each part 256-byte aligned.
extern "C" size_t dspark_l1_loss_workspace_bytes(int B, int A, int gamma, int V, int dtype) {
  if (B <= 0 || A <= 0 || gamma <= 0 || V <= 0) return 0;
  if (dtype != DSPARK_BF16 && dtype != DSPARK_F32) return 0;
  return layout((int64_t)B * A * gamma, geometry(V, dtype)).total;
}

extern "C" int dspark_l1_loss(const void* draft_logits, const void* target_logits, const uint8_t* eval_mask,
                              float decay, float* loss, float* row_l1, float* grad, float* tau_greedy, int B,
                              int A, int gamma, int V, int dtype, void* ws, size_t ws_bytes, void* stream) {
  using namespace dspark_host;
  if (B < 0 || A < 0 || gamma < 0) return fail(DSPARK_ERR_INVALID_ARG, "l1_loss: negative dimension");
  if (dtype != DSPARK_BF16 && dtype != DSPARK_F32)
    return fail(DSPARK_ERR_INVALID_ARG, "l1_loss: unknown dtype %d", dtype);
  if (V < 1) return fail(DSPARK_ERR_INVALID_ARG, "l1_loss: V must be >= 1 (got %d)", V);
  if (gamma > 1024) return fail(DSPARK_ERR_INVALID_ARG, "l1_loss: gamma > 1024");
  if (!(decay > 0.f) || decay == INFINITY)
    return fail(DSPARK_ERR_INVALID_ARG, "l1_loss: decay must be finite and > 0");
  const int64_t rows = (int64_t)B * A * gamma;
  if (!loss) return fail(DSPARK_ERR_INVALID_ARG, "l1_loss: null loss pointer");
  hipStream_t s = (hipStream_t)stream;
  if (rows == 0) {
    hipLaunchKernelGGL(l1_finalize_kernel, dim3(1), dim3(kThreads), 0, s, (const float*)nullptr,
                       (const float*)nullptr, (const float*)nullptr, (const uint8_t*)nullptr, loss,
                       (float*)nullptr, (int64_t)0, 1);
    return check_launch("l1_loss");
  }
  if (!draft_logits || !target_logits) return fail(DSPARK_ERR_INVALID_ARG, "l1_loss: null required pointer");
  const Geometry geo = geometry(V, dtype);
  const Layout L = layout(rows, geo);
  if (ws_bytes < L.total || !ws)
    return fail(DSPARK_ERR_WORKSPACE, "l1_loss: workspace %zu bytes < %zu", ws_bytes, L.total);
  char* wsb = (char*)ws;
  float* coef = (float*)(wsb + L.coef);
  float* l1 = row_l1 ? row_l1 : (float*)(wsb + L.l1);
  float* greedy = (float*)(wsb + L.greedy);
  const int cus = device_cu_count();
  if (cus <= 0) return fail(DSPARK_ERR_HIP, "l1_loss: device query failed");
  hipLaunchKernelGGL(l1_coef_kernel, dim3(1), dim3(kThreads), 0, s, eval_mask, coef, rows, gamma, decay);
  const bool bf = dtype == DSPARK_BF16;
  const int el = bf ? 8 : 4;
  const bool vec = V % el == 0 && (uintptr_t)draft_logits % 16 == 0 && (uintptr_t)target_logits % 16 == 0;
  // cluster path: 16-byte rows (and gradient), V within 128 slices
  int64_t ncl = 0;
  const void* ckern = nullptr;
  if (vec && geo.G > 0 && (uintptr_t)grad % 16 == 0) {
    ckern = bf ? (grad ? (const void*)l1_cluster_kernel<true, true> : (const void*)l1_cluster_kernel<true, false>)
               : (grad ? (const void*)l1_cluster_kernel<false, true> : (const void*)l1_cluster_kernel<false, false>);
    const int cap = cluster::cluster_capacity(ckern, kCThreads, "l1_loss");
    if (cap <= 0) return fail(DSPARK_ERR_HIP, "l1_loss: occupancy query failed");
    ncl = std::min<int64_t>(cap / geo.G, max_clusters(rows, geo.G));
  }
  if (ncl >= 1) {
    u32x4* rec = (u32x4*)(wsb + L.rec);
    u32x4* slots = (u32x4*)(wsb + L.slots);
    uint32_t* sslots = (uint32_t*)(wsb + L.sslots);
    int32_t* err = (int32_t*)(wsb + L.err);
    // slots (epoch 0 = empty) and the error word start at zero: a fill kernel,
    // not a memset node, so the sequence stays safe under graph capture
    const int64_t nwords = (int64_t)(L.total - L.slots) / 4;
    hipLaunchKernelGGL(l1_zero_u32_kernel, dim3((unsigned)((nwords + 255) / 256)), dim3(256), 0, s,
                       (uint32_t*)slots, nwords);
    const char* dp = (const char*)draft_logits;
    const char* tp = (const char*)target_logits;
    int64_t rows_arg = rows;
    int Varg = V, vpr = geo.vec_per_row, G = geo.G, ncl_arg = (int)ncl;
    unsigned spin = wait_limit();
    void* args[] = {(void*)&dp, (void*)&tp, (void*)&coef, (void*)&grad, (void*)&rec, (void*)&rows_arg,
                    (void*)&Varg, (void*)&vpr, (void*)&G, (void*)&ncl_arg, (void*)&slots, (void*)&sslots,
                    (void*)&err, (void*)&spin};
    if (getenv("DSPARK_VERBOSE"))
      fprintf(stderr, "[dspark] l1_loss: %d CUs, G=%d, clusters=%lld\n", cus, G, (long long)ncl);
    hipError_t e = hipLaunchCooperativeKernel(ckern, dim3((unsigned)(ncl * G)), dim3(kCThreads), args, 0, s);
    if (e != hipSuccess) return fail(DSPARK_ERR_HIP, "l1_loss: cooperative launch: %s", hipGetErrorString(e));
    hipLaunchKernelGGL(l1_cluster_finalize_kernel, dim3((unsigned)((rows + kFinRows - 1) / kFinRows)),
                       dim3(64 * kFinRows), 0, s, (const u32x4*)rec, G, l1, greedy, rows);
  } else {
    const unsigned grid = (unsigned)(rows < cus ? rows : cus);
    if (bf) {
      if (vec) hipLaunchKernelGGL((l1_rows_kernel<true, true>), dim3(grid), dim3(kThreads), 0, s, draft_logits, target_logits, coef, l1, greedy, grad, rows, V);
      else hipLaunchKernelGGL((l1_rows_kernel<true, false>), dim3(grid), dim3(kThreads), 0, s, draft_logits, target_logits, coef, l1, greedy, grad, rows, V);
    } else {
      if (vec) hipLaunchKernelGGL((l1_rows_kernel<false, true>), dim3(grid), dim3(kThreads), 0, s, draft_logits, target_logits, coef, l1, greedy, grad, rows, V);
      else hipLaunchKernelGGL((l1_rows_kernel<false, false>), dim3(grid), dim3(kThreads), 0, s, draft_logits, target_logits, coef, l1, greedy, grad, rows, V);
    }
  }
  hipLaunchKernelGGL(l1_finalize_kernel, dim3(1), dim3(kThreads), 0, s, (const float*)coef, (const float*)l1,
                     (const float*)greedy, eval_mask, loss, tau_greedy, rows, gamma);
  return check_launch("l1_loss");
}
