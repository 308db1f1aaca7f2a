// TV-distance accept rate (page 1, "03 · DSpark 建模", §3.9, the paper's
// Eq. 8; page 2 §3.5 / §3.8.3) and tau (page 1 §3.10).
//
//   accept = clamp(1 - 1/2 sum_v |p_v - q_v|, 0, 1),  p = softmax(draft), q = softmax(target)
//
// computed through the equivalent form 1 - TV(p, q) = sum_v min(p_v, q_v)
// (valid because both distributions sum to one): with
// y_v = x_v * log2(e) - (M * log2(e) + log2 S), p_v = 2^{y_v}, and since 2^y
// is monotonic, min(p_v, q_v) = 2^{min(yd_v, yt_v)} costs one exponential per
// element pair instead of two.
//
// HBM-bound design for gfx950: a row (2 x V logits) is split over a cluster of
// G workgroups.  Each workgroup loads its slice of both tensors ONCE into
// registers (16-byte coalesced loads), computes its local max and sum, and the
// cluster exchanges (max, sum) through a few bytes of global memory; pass two
// runs on the register-resident slice and the last workgroup of the cluster to
// finish folds the partial sums (in fixed order, so results are deterministic)
// and writes the accept rate.  The grid is persistent and launched
// cooperatively so every workgroup of a cluster is co-resident; every wait is
// bounded.  The maximum of bf16 data is taken on the raw bits with packed
// 16-bit integer max/min (two elements per instruction).
#include <stdlib.h>

#include <map>
#include <mutex>
#include <utility>

#include "common.h"

using namespace dspark;

namespace {

constexpr int kThreads = 256;
constexpr int kMaxVec = 5;  // 16-byte vectors per thread per tensor (152 VGPRs: 3 WGs per CU)
constexpr float kLog2e = 1.4426950408889634f;
constexpr unsigned kSpinLimit = 1u << 26;  // bounded wait (~seconds), then flag and go on

typedef short short2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Reduce two floats over the workgroup (max or sum); all threads get the result.
template <bool kMax>
__device__ __forceinline__ void block_reduce2(float& a, float& b, float* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  a = kMax ? wave_max(a) : wave_sum(a);
  b = kMax ? wave_max(b) : wave_sum(b);
  __syncthreads();  // red[] may still be read by the previous reduction
  if (lane == 0) { red[w] = a; red[4 + w] = b; }
  __syncthreads();
  if (kMax) {
    a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    b = fmaxf(fmaxf(red[4], red[5]), fmaxf(red[6], red[7]));
  } else {
    a = (red[0] + red[1]) + (red[2] + red[3]);
    b = (red[4] + red[5]) + (red[6] + red[7]);
  }
}

// Largest value among the bf16 pairs reduced with packed int16 max/min.
__device__ __forceinline__ float bf16_pair_max(short2v mx, short2v mn) {
  const short hmax = mx.x > mx.y ? mx.x : mx.y;
  if (hmax >= 0) return __uint_as_float((uint32_t)(uint16_t)hmax << 16);
  // every element is negative: the largest is the one of smallest magnitude,
  // whose sign-magnitude pattern is the smallest as int16
  const short hmin = mn.x < mn.y ? mn.x : mn.y;
  return __uint_as_float((uint32_t)(uint16_t)hmin << 16);
}

template <bool kBf16>
__device__ __forceinline__ float vec_max(const u32x4* v, int nvalid) {
  if (kBf16) {
    short2v mx = {(short)-32768, (short)-32768}, mn = {(short)32767, (short)32767};
#pragma unroll
    for (int i = 0; i < kMaxVec; ++i) {
      if (i < nvalid) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          short2v s = __builtin_bit_cast(short2v, v[i][c]);
          mx = __builtin_elementwise_max(mx, s);
          mn = __builtin_elementwise_min(mn, s);
        }
      }
    }
    return nvalid > 0 ? bf16_pair_max(mx, mn) : -INFINITY;
  } else {
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < kMaxVec; ++i)
      if (i < nvalid)
#pragma unroll
        for (int c = 0; c < 4; ++c) m = fmaxf(m, __uint_as_float(v[i][c]));
    return m;
  }
}

// sum of 2^{x*log2e - mL} over the thread's elements
template <bool kBf16>
__device__ __forceinline__ float vec_sumexp(const u32x4* v, int nvalid, float mL) {
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxVec; ++i) {
    if (i < nvalid) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t w = v[i][c];
        if (kBf16) {
          s0 += exp2_fast(fmaf(bf16lo(w), kLog2e, -mL));
          s1 += exp2_fast(fmaf(bf16hi(w), kLog2e, -mL));
        } else {
          s0 += exp2_fast(fmaf(__uint_as_float(w), kLog2e, -mL));
        }
      }
    }
  }
  return s0 + s1;
}

// sum of 2^{min(yd, yt)}
template <bool kBf16>
__device__ __forceinline__ float vec_summin(const u32x4* dv, const u32x4* tv, int nvalid,
                                            float offd, float offt) {
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxVec; ++i) {
    if (i < nvalid) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t a = dv[i][c], b = tv[i][c];
        if (kBf16) {
          s0 += exp2_fast(fminf(fmaf(bf16lo(a), kLog2e, -offd), fmaf(bf16lo(b), kLog2e, -offt)));
          s1 += exp2_fast(fminf(fmaf(bf16hi(a), kLog2e, -offd), fmaf(bf16hi(b), kLog2e, -offt)));
        } else {
          s0 += exp2_fast(fminf(fmaf(__uint_as_float(a), kLog2e, -offd),
                                fmaf(__uint_as_float(b), kLog2e, -offt)));
        }
      }
    }
  }
  return s0 + s1;
}

// ---- cluster exchange without fences.  Every published float travels with
// its iteration number ("epoch") in one 64-bit word written and read with
// relaxed agent-scope atomics (coherent across the XCDs' L2s), so a reader
// that sees the right epoch also sees the value: no release/acquire cache
// maintenance per poll.  Epochs start at 1; the slots are zeroed per launch.
__device__ __forceinline__ void publish(uint64_t* slot, float v, uint32_t epoch) {
  const uint64_t w = ((uint64_t)epoch << 32) | __float_as_uint(v);
  __hip_atomic_store(slot, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Bounded wait for one slot; NaN (and a flag) on time-out.
__device__ __forceinline__ float collect(uint64_t* slot, uint32_t epoch, int32_t* err, bool& ok) {
  unsigned n = 0;
  for (;;) {
    const uint64_t w = __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((uint32_t)(w >> 32) == epoch) return __uint_as_float((uint32_t)w);
    if (!ok || ++n > kSpinLimit) {
      if (ok) atomicOr(err, 1);
      ok = false;
      return NAN;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// Workspace per cluster: slots[2 phases][2 parities][G][4] 64-bit words.
template <bool kBf16>
__global__ __launch_bounds__(kThreads) void tv_cluster_kernel(
    const u32x4* __restrict__ d, const u32x4* __restrict__ t, float* __restrict__ accept,
    int64_t rows, int vec_per_row, int vec_per_wg, int G, int nclusters,
    uint64_t* __restrict__ slots, int32_t* __restrict__ err) {
  __shared__ float red[8];
  __shared__ float bcast[4];
  const int cl = blockIdx.x / G, g = blockIdx.x % G;
  const int v0 = g * vec_per_wg;
  const int v1 = min(v0 + vec_per_wg, vec_per_row);
  const int first = v0 + (int)threadIdx.x;
  const int nvalid = first < v1 ? min(kMaxVec, (v1 - first + kThreads - 1) / kThreads) : 0;
  uint64_t* cslots = slots + (size_t)cl * 16 * G;
  int it = 0;
  bool ok = true;  // after one timed-out wait this workgroup stops waiting
  for (int64_t row = cl; row < rows; row += nclusters, ++it) {
    const uint32_t epoch = (uint32_t)it + 1u;
    uint64_t* slotA = cslots + (0 * 2 + (it & 1)) * G * 4;
    uint64_t* slotB = cslots + (1 * 2 + (it & 1)) * G * 4;
    const u32x4* dr = d + row * vec_per_row;
    const u32x4* tr = t + row * vec_per_row;
    u32x4 dv[kMaxVec], tv[kMaxVec];
#pragma unroll
    for (int i = 0; i < kMaxVec; ++i) {
      if (i < nvalid) {
        dv[i] = __builtin_nontemporal_load(dr + first + i * kThreads);
        tv[i] = __builtin_nontemporal_load(tr + first + i * kThreads);
      }
    }
    // ---- local statistics (max, then sum relative to the workgroup max)
    float md = vec_max<kBf16>(dv, nvalid), mt = vec_max<kBf16>(tv, nvalid);
    block_reduce2<true>(md, mt, red);
    float sd = vec_sumexp<kBf16>(dv, nvalid, md * kLog2e);
    float st = vec_sumexp<kBf16>(tv, nvalid, mt * kLog2e);
    block_reduce2<false>(sd, st, red);
    // ---- cluster exchange of (max, sum) for both tensors
    float Md = md, Sd = sd, Mt = mt, St = st;
    if (G > 1) {
      if (threadIdx.x < 4) {
        const float mine = threadIdx.x == 0 ? md : threadIdx.x == 1 ? sd : threadIdx.x == 2 ? mt : st;
        publish(slotA + g * 4 + threadIdx.x, mine, epoch);
      }
      // lanes j < G of wave 0 collect workgroup j's statistics
      if (threadIdx.x < 64) {
        const int j = threadIdx.x;
        float mj = -INFINITY, sj = 0.f, nj = -INFINITY, tj = 0.f;
        if (j < G) {
          mj = collect(slotA + j * 4 + 0, epoch, err, ok);
          sj = collect(slotA + j * 4 + 1, epoch, err, ok);
          nj = collect(slotA + j * 4 + 2, epoch, err, ok);
          tj = collect(slotA + j * 4 + 3, epoch, err, ok);
        }
        float a = mj, b = nj;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          a = fmaxf(a, __shfl_xor(a, o, kWave));
          b = fmaxf(b, __shfl_xor(b, o, kWave));
        }
        float sa = sj > 0.f ? sj * exp2_fast((mj - a) * kLog2e) : 0.f;
        float sb = tj > 0.f ? tj * exp2_fast((nj - b) * kLog2e) : 0.f;
        // fixed-order sum over j (lanes) so every workgroup gets identical bits
        float SA = 0.f, SB = 0.f;
        for (int q = 0; q < G; ++q) {
          SA += __shfl(sa, q, kWave);
          SB += __shfl(sb, q, kWave);
        }
        const bool poisoned = __any(!ok);  // a timed-out wait poisons the row
        if (j == 0) {
          bcast[0] = poisoned ? NAN : a;
          bcast[1] = SA; bcast[2] = b; bcast[3] = SB;
        }
      }
      __syncthreads();
      Md = bcast[0]; Sd = bcast[1]; Mt = bcast[2]; St = bcast[3];
    }
    const float offd = Md * kLog2e + __builtin_amdgcn_logf(Sd);
    const float offt = Mt * kLog2e + __builtin_amdgcn_logf(St);
    // ---- pass two on the register-resident slice
    float part = vec_summin<kBf16>(dv, tv, nvalid, offd, offt);
    float dummy = 0.f;
    block_reduce2<false>(part, dummy, red);
    if (G == 1) {
      if (threadIdx.x == 0) accept[row] = fminf(fmaxf(part, 0.f), 1.f);
    } else {
      if (threadIdx.x == 0) publish(slotB + g * 4, part, epoch);
      // one workgroup per row (rotating) folds the partial sums in fixed order
      if (g == it % G && threadIdx.x < 64) {
        const int j = threadIdx.x;
        const float pj = j < G ? collect(slotB + j * 4, epoch, err, ok) : 0.f;
        float s = 0.f;
        for (int q = 0; q < G; ++q) s += __shfl(pj, q, kWave);
        if (j == 0) accept[row] = fminf(fmaxf(s, 0.f), 1.f);
      }
    }
  }
}

__global__ void zero_u32_kernel(unsigned* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// Fallback for rows that are not 16-byte aligned (V not a multiple of the
// vector width): one workgroup per row, three streaming passes over global
// memory.  Correctness path only.
template <bool kBf16>
__global__ __launch_bounds__(kThreads) void tv_rowwise_kernel(const void* __restrict__ d,
                                                              const void* __restrict__ t,
                                                              float* __restrict__ accept,
                                                              int64_t rows, int V) {
  __shared__ float red[8];
  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    auto ld = [&](const void* p, int v) -> float {
      if (kBf16) {
        const uint16_t h = ((const uint16_t*)p)[row * V + v];
        return __uint_as_float((uint32_t)h << 16);
      }
      return ((const float*)p)[row * V + v];
    };
    float md = -INFINITY, mt = -INFINITY;
    for (int v = threadIdx.x; v < V; v += kThreads) { md = fmaxf(md, ld(d, v)); mt = fmaxf(mt, ld(t, v)); }
    block_reduce2<true>(md, mt, red);
    float sd = 0.f, st = 0.f;
    for (int v = threadIdx.x; v < V; v += kThreads) {
      sd += exp2_fast((ld(d, v) - md) * kLog2e);
      st += exp2_fast((ld(t, v) - mt) * kLog2e);
    }
    block_reduce2<false>(sd, st, red);
    const float offd = md * kLog2e + __builtin_amdgcn_logf(sd);
    const float offt = mt * kLog2e + __builtin_amdgcn_logf(st);
    float s = 0.f, dummy = 0.f;
    for (int v = threadIdx.x; v < V; v += kThreads)
      s += exp2_fast(fminf(fmaf(ld(d, v), kLog2e, -offd), fmaf(ld(t, v), kLog2e, -offt)));
    block_reduce2<false>(s, dummy, red);
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

struct Plan {
  bool vec;
  int vec_per_row, G, vec_per_wg, nclusters;
};

int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  return cus;
}

// Co-resident workgroups of `kernel` on the current device, cached per
// (device, kernel): the occupancy query is far slower than a launch.
int device_wg_capacity(const void* kernel) {
  static std::mutex mu;
  static std::map<std::pair<int, const void*>, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find({dev, kernel});
  if (it != cache.end()) return it->second;
  int cus = 0, per = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, kThreads, 0) != hipSuccess) return -1;
  cache[{dev, kernel}] = cus * per;
  return cus * per;
}

Plan make_plan(int64_t rows, int V, int dtype, int capacity) {
  Plan p{};
  const int epv = dtype == DSPARK_BF16 ? 8 : 4;
  p.vec = (V % epv) == 0;
  if (!p.vec) return p;
  p.vec_per_row = V / epv;
  p.G = (p.vec_per_row + kThreads * kMaxVec - 1) / (kThreads * kMaxVec);
  p.vec_per_wg = (p.vec_per_row + p.G - 1) / p.G;
  int64_t cl = capacity > 0 ? capacity / p.G : 1;
  if (cl > rows) cl = rows;
  if (cl < 1) cl = 1;
  p.nclusters = (int)cl;
  return p;
}

}  // namespace

extern "C" size_t dspark_accept_rate_workspace_bytes(int B, int A, int gamma, int V, int dtype) {
  if (B < 0 || A < 0 || gamma < 0 || V < 0) return 0;
  // Upper bound independent of the device: one cluster per row at most and
  // at most 16 workgroups per compute unit on 256 compute units.
  const int64_t rows = (int64_t)B * A * gamma;
  const int epv = dtype == DSPARK_BF16 ? 8 : 4;
  const int64_t vpr = V / epv > 0 ? V / epv : 1;
  const int64_t G = (vpr + kThreads * kMaxVec - 1) / (kThreads * kMaxVec);
  int64_t cl = (256 * 16) / (G > 0 ? G : 1);
  if (cl > rows) cl = rows;
  if (cl < 1) cl = 1;
  return (size_t)(cl * 16 * G * sizeof(uint64_t) + 64);
}

extern "C" int dspark_accept_rate(const void* draft_logits, const void* target_logits,
                                  float* accept, const uint8_t* eval_mask, float* tau, int B,
                                  int A, int gamma, int V, int dtype, void* ws, size_t ws_bytes,
                                  void* stream) {
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
  const void* kern = bf ? (const void*)tv_cluster_kernel<true> : (const void*)tv_cluster_kernel<false>;
  const int cap = device_wg_capacity(kern);
  if (cap <= 0) return fail(DSPARK_ERR_HIP, "accept_rate: occupancy query failed");
  Plan p = make_plan(rows, V, dtype, cap);
  if (p.vec && aligned) {
    // the workspace bound assumes at most 16 workgroups per CU on 256 CUs
    const int64_t max_cl = (256 * 16) / p.G;
    if (p.nclusters > max_cl) p.nclusters = (int)max_cl;
    uint64_t* slots = (uint64_t*)ws;
    const int64_t nslot = (int64_t)p.nclusters * 16 * p.G;
    int32_t* err = (int32_t*)(slots + nslot);  // one spare word after the slots
    // slots (epoch 0 = empty) and the error word start at zero: a fill
    // kernel, not a memset node, so the sequence stays safe under graph capture
    const int64_t nwords = nslot * 2 + 1;
    hipLaunchKernelGGL(zero_u32_kernel, dim3((unsigned)((nwords + 255) / 256)), dim3(256), 0, s,
                       (unsigned*)ws, (int)nwords);
    const u32x4* dp = (const u32x4*)draft_logits;
    const u32x4* tp = (const u32x4*)target_logits;
    int64_t rows_arg = rows;
    int vpr = p.vec_per_row, vpw = p.vec_per_wg, G = p.G, ncl = p.nclusters;
    void* args[] = {(void*)&dp, (void*)&tp, (void*)&accept, (void*)&rows_arg, (void*)&vpr,
                    (void*)&vpw, (void*)&G, (void*)&ncl, (void*)&slots, (void*)&err};
    if (getenv("DSPARK_VERBOSE"))
      fprintf(stderr, "[dspark] accept_rate: capacity %d WGs (%d CUs), G=%d, clusters=%d, vec/row=%d\n",
              cap, device_cus(), p.G, p.nclusters, p.vec_per_row);
    hipError_t e = hipLaunchCooperativeKernel(kern, dim3((unsigned)(p.nclusters * p.G)),
                                              dim3(kThreads), args, 0, s);
    if (e != hipSuccess)
      return fail(DSPARK_ERR_HIP, "accept_rate: cooperative launch: %s", hipGetErrorString(e));
  } else {
    int64_t grid = rows < 65536 ? rows : 65536;
    if (bf)
      hipLaunchKernelGGL(tv_rowwise_kernel<true>, dim3((unsigned)grid), dim3(kThreads), 0, s,
                         draft_logits, target_logits, accept, rows, V);
    else
      hipLaunchKernelGGL(tv_rowwise_kernel<false>, dim3((unsigned)grid), dim3(kThreads), 0, s,
                         draft_logits, target_logits, accept, rows, V);
  }
  if (tau) {
    const int64_t nb = (int64_t)B * A;
    hipLaunchKernelGGL(tau_kernel, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, s, accept,
                       eval_mask, tau, nb, gamma);
  }
  return check_launch("accept_rate");
}
