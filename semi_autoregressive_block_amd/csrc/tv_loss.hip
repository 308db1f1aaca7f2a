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
// gfx950 design: one 16-wave workgroup per row and one workgroup per compute
// unit, so the rows in flight (256 x 2 x V x 2 bytes, 155 MB for bf16 at
// V = 151936) stay in the 256 MB last-level cache between the passes over a
// row: pass one takes each thread's online (max, sum of exponentials) and
// argmax in one sweep, pass two the row's L1 distance and sum_u s_u p_u, and
// pass three (only when the gradient is wanted) writes c p (s - S).  Rows
// are read with 16-byte loads when the row length and the buffers allow it.
// Every reduction runs in a fixed order, so results are deterministic.
#include <limits.h>

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

// c[n] = w_k m_n / sum(w m) with w_k = exp(-k / decay); one workgroup, fixed
// summation order.  All zeros when no position is valid.
__global__ __launch_bounds__(kThreads) void l1_coef_kernel(const uint8_t* __restrict__ m, float* __restrict__ coef,
                                                           int64_t rows, int gamma, float decay) {
  __shared__ float red[1][kWaves];
  float part[1] = {0.f};
  for (int64_t n = threadIdx.x; n < rows; n += kThreads)
    if (!m || m[n]) part[0] += expf(-(float)(n % gamma) / decay);
  block_sum(part, red);
  const float inv = part[0] > 0.f ? 1.f / part[0] : 0.f;
  for (int64_t n = threadIdx.x; n < rows; n += kThreads)
    coef[n] = (!m || m[n]) ? expf(-(float)(n % gamma) / decay) * inv : 0.f;
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

}  // namespace

// Workspace: c [rows] | l1 [rows] | greedy [rows], float32, 256-byte aligned.
extern "C" size_t dspark_l1_loss_workspace_bytes(int B, int A, int gamma) {
  if (B <= 0 || A <= 0 || gamma <= 0) return 0;
  return 3 * dspark_host::align_up((size_t)B * A * gamma * sizeof(float), 256);
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
  const size_t need = dspark_l1_loss_workspace_bytes(B, A, gamma);
  if (ws_bytes < need || !ws) return fail(DSPARK_ERR_WORKSPACE, "l1_loss: workspace %zu bytes < %zu", ws_bytes, need);
  const size_t slab = align_up((size_t)rows * sizeof(float), 256);
  float* coef = (float*)ws;
  float* l1 = row_l1 ? row_l1 : (float*)((char*)ws + slab);
  float* greedy = (float*)((char*)ws + 2 * slab);
  const int cus = device_cu_count();
  if (cus <= 0) return fail(DSPARK_ERR_HIP, "l1_loss: device query failed");
  hipLaunchKernelGGL(l1_coef_kernel, dim3(1), dim3(kThreads), 0, s, eval_mask, coef, rows, gamma, decay);
  const bool bf = dtype == DSPARK_BF16;
  const int el = bf ? 8 : 4;
  const bool vec = V % el == 0 && (uintptr_t)draft_logits % 16 == 0 && (uintptr_t)target_logits % 16 == 0;
  const unsigned grid = (unsigned)(rows < cus ? rows : cus);
  if (bf) {
    if (vec) hipLaunchKernelGGL((l1_rows_kernel<true, true>), dim3(grid), dim3(kThreads), 0, s, draft_logits, target_logits, coef, l1, greedy, grad, rows, V);
    else hipLaunchKernelGGL((l1_rows_kernel<true, false>), dim3(grid), dim3(kThreads), 0, s, draft_logits, target_logits, coef, l1, greedy, grad, rows, V);
  } else {
    if (vec) hipLaunchKernelGGL((l1_rows_kernel<false, true>), dim3(grid), dim3(kThreads), 0, s, draft_logits, target_logits, coef, l1, greedy, grad, rows, V);
    else hipLaunchKernelGGL((l1_rows_kernel<false, false>), dim3(grid), dim3(kThreads), 0, s, draft_logits, target_logits, coef, l1, greedy, grad, rows, V);
  }
  hipLaunchKernelGGL(l1_finalize_kernel, dim3(1), dim3(kThreads), 0, s, (const float*)coef, (const float*)l1,
                     (const float*)greedy, eval_mask, loss, tau_greedy, rows, gamma);
  return check_launch("l1_loss");
}
