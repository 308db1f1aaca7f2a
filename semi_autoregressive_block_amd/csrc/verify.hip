// Lossless verify step: rejection sampling of a drafted block against the
// target model (page 3, "如何评价 DeepSeek 发布 DSpark？哪些亮点值得关注？", the
// speculative-decoding primer;
// page 4, "DSpark 深度解读", §1.2).  The pages give the outline (accept the
// prefix consistent with P from left to right, cut at the first failure
// and draw that position again from the target, output distribution
// unchanged); the steps are the published speculative-sampling rule
// (Leviathan, Kalman, Matias, ICML 2023; Chen et al. 2023):
//
//   q_k = softmax(draft[k] / T), p_k = softmax(target[k] / T)
//   keep x_k while u_k < p_k(x_k) / q_k(x_k)
//   first rejected k: draw from max(0, p_k - q_k) (normalised)
//   all K kept: draw one more token from p_K
//   T = 0: keep x_k while it is the target's argmax; the extra token is the
//   target's argmax at the stopping position
//
// Random numbers: Philox4x32-10 keyed by the seed; u_k is word 0 at counter
// (k, 0, row, 2) as ((x >> 9) + 1/2) 2^-23; the draws are Gumbel-max with
// word v & 3 at counter (v >> 2, k, row, 1) (streams apart from the draft
// sampler's stream 0).
//
// Three kernels: per (row, position) softmax statistics (one workgroup
// each, so the whole chip streams the logits), a per-row left-to-right
// decision, then one pass over the vocabulary at each row's stopping
// position with the argmax folded through 64-bit (value, index) keys.
#include "common.h"
#include "philox.h"

using namespace dspark;

namespace {

constexpr int kThreads = 256;
constexpr int kStat = 8;  // floats per (row, position): m_t, s_t, m_d, s_d, argmax_t bits (3 spare)

struct Soft {
  float m, s;
};

// Running (max, sum of 2^(y - max)) with one exponential per element; the
// statistics pass works on y = logits * log2(e) / T (base 2: one v_exp_f32
// per element) and converts the maximum back to natural-log scale at the
// end (the sum is the same in both bases).  The running maximum starts at
// -FLT_MAX, not -inf, so a masked logit (-inf) adds 2^-inf = 0 even before
// the first finite one (-inf - -inf would be NaN), at no extra instruction.
constexpr float kSoftInit = -3.402823466e38f;
constexpr float kLog2eF = 1.4426950408889634f, kLn2F = 0.69314718055994531f;
__device__ __forceinline__ void soft_add2(Soft& a, float y) {
  if (y > a.m) {
    a.s = a.s * exp2f(a.m - y) + 1.f;
    a.m = y;
  } else {
    a.s += exp2f(y - a.m);
  }
}
__device__ __forceinline__ Soft soft_merge2(Soft a, Soft b) {
  const float m = fmaxf(a.m, b.m);
  if (m == -INFINITY) return {m, 0.f};
  return {m, a.s * exp2f(a.m - m) + b.s * exp2f(b.m - m)};
}

template <int NT = kThreads, typename T, typename F>
__device__ __forceinline__ T block_reduce(T v, F op, T* lds) {
  for (int off = 32; off > 0; off >>= 1) {
    T o;
    if constexpr (sizeof(T) == 8) {
      uint64_t b = __builtin_bit_cast(uint64_t, v);
      const uint32_t lo = __shfl_xor((uint32_t)b, off, kWave), hi = __shfl_xor((uint32_t)(b >> 32), off, kWave);
      o = __builtin_bit_cast(T, ((uint64_t)hi << 32) | lo);
    } else {
      o = __builtin_bit_cast(T, __shfl_xor(__builtin_bit_cast(uint32_t, v), off, kWave));
    }
    v = op(v, o);
  }
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) lds[w] = v;
  __syncthreads();
  v = lds[0];
  for (int i = 1; i < NT / 64; ++i) v = op(v, lds[i]);
  return v;
}

// Statistics of position k (blockIdx.x) of row blockIdx.y over the scaled
// logits y = logits / T (T = 0: only the target's argmax).  With 16-byte
// rows (vec) each thread takes kBatch vectors of the target row and as many
// of the draft row per step, all loads issued before any is used (a single
// load in flight per thread left the stream latency-bound), then folds each
// row's batch into its running (max, sum) with one rescale per batch and
// one exponential per element.
constexpr int kBatch = 8;
__device__ __forceinline__ void soft_add_batch(Soft& a, const f32x4* y, float sc) {
  float m = a.m;
#pragma unroll
  for (int b = 0; b < kBatch; ++b)
#pragma unroll
    for (int e = 0; e < 4; ++e) m = fmaxf(m, y[b][e] * sc);
  a.s *= exp2f(a.m - m);  // m >= a.m > -inf
  a.m = m;
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int b = 0; b < kBatch; ++b) {
    s0 += exp2f(fmaf(y[b][0], sc, -m)) + exp2f(fmaf(y[b][1], sc, -m));
    s1 += exp2f(fmaf(y[b][2], sc, -m)) + exp2f(fmaf(y[b][3], sc, -m));
  }
  a.s += s0 + s1;
}

__global__ __launch_bounds__(kThreads) void verify_stats_kernel(const float* __restrict__ draft,
                                                                const float* __restrict__ target, int K, int V,
                                                                float invT, int greedy, int vec,
                                                                float* __restrict__ stats) {
  __shared__ uint64_t lds64[kThreads / 64];
  __shared__ Soft ldss[kThreads / 64];
  const int k = blockIdx.x, row = blockIdx.y;
  const float* t = target + ((int64_t)row * (K + 1) + k) * V;
  const bool with_d = !greedy && k < K;
  const float* d = draft + ((int64_t)row * K + (k < K ? k : 0)) * V;
  constexpr float kLog2e = 1.4426950408889634f, kLn2 = 0.69314718055994531f;
  const float sc = invT * kLog2e;
  Soft st{kSoftInit, 0.f}, sd{kSoftInit, 0.f};
  float bv = -INFINITY;  // this thread's first maximum (indices rise along its scan)
  uint32_t bi = 0xffffffffu;
  const int nv = vec ? V / 4 : 0;
  const f32x4 none = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  for (int c0 = threadIdx.x; c0 < nv; c0 += kThreads * kBatch) {
    f32x4 yt[kBatch], yd[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int c = c0 + b * kThreads;
      yt[b] = c < nv ? *(const f32x4*)(t + 4 * c) : none;
      yd[b] = with_d && c < nv ? *(const f32x4*)(d + 4 * c) : none;
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (yt[b][e] > bv) { bv = yt[b][e]; bi = (uint32_t)(4 * (c0 + b * kThreads) + e); }
    if (!greedy) soft_add_batch(st, yt, sc);
    if (with_d) soft_add_batch(sd, yd, sc);
  }
  for (int v = 4 * nv + threadIdx.x; v < V; v += kThreads) {
    const float y = t[v];
    if (y > bv) { bv = y; bi = (uint32_t)v; }
    if (!greedy) soft_add2(st, y * sc);
    if (with_d) soft_add2(sd, d[v] * sc);
  }
  uint64_t best = bi == 0xffffffffu ? 0ull : argmax_key(bv, bi);
  best = block_reduce(best, [](uint64_t a, uint64_t b) { return a > b ? a : b; }, lds64);
  float* out = stats + ((int64_t)row * (K + 1) + k) * kStat;
  if (!greedy) st = block_reduce(st, soft_merge2, ldss);
  if (with_d) sd = block_reduce(sd, soft_merge2, ldss);
  st.m *= kLn2;
  sd.m *= kLn2;
  if (threadIdx.x == 0) {
    out[0] = st.m; out[1] = st.s; out[2] = sd.m; out[3] = sd.s;
    out[4] = __uint_as_float(argmax_key_index(best));
  }
}

// The left-to-right acceptance test of every request: its first rejected position.
__global__ __launch_bounds__(64) void verify_decide_kernel(const float* __restrict__ draft,
                                                            const float* __restrict__ target,
                                                            const int32_t* __restrict__ tokens,
                                                            const float* __restrict__ stats, int R, int K, int V,
                                                            float invT, int greedy, uint32_t slo, uint32_t shi,
                                                            int32_t* __restrict__ n_acc, int32_t* __restrict__ pos_out,
                                                            int32_t* __restrict__ next_token,
                                                            int32_t* __restrict__ status, uint64_t* __restrict__ keys) {
  // 16 lanes per request (four requests per wave), lane p testing position c + p of each
  // 16-position chunk c: every position's loads are in flight at once, and a ballot finds the
  // request's first rejection.  A position's test is the same arithmetic as a sequential scan.
  // Every draft token is range-checked, also those past the stop.
  const int lane = threadIdx.x, sub = lane >> 4, p = lane & 15;
  const int row = blockIdx.x * 4 + sub;
  const bool live = row < R;
  int stop = -1;  // the request's first rejected position once found (the same in its 16 lanes)
  bool bad_any = false;
  for (int c = 0; c < K; c += 16) {
    const int pos = c + p;
    const bool inrange = live && pos < K;
    int x = 0;
    if (inrange) {
      x = tokens[(int64_t)row * K + pos];
      if (x < 0 || x >= V) {
        bad_any = true;
        x = 0;
      }
    }
    bool reject = false;
    if (inrange && stop < 0) {
      const float* s = stats + ((int64_t)row * (K + 1) + pos) * kStat;
      if (greedy) {
        reject = (uint32_t)x != __float_as_uint(s[4]);
      } else {
        const float lp = target[((int64_t)row * (K + 1) + pos) * V + x] * invT - s[0] - logf(s[1]);
        const float lq = draft[((int64_t)row * K + pos) * V + x] * invT - s[2] - logf(s[3]);
        const u32x4 w = philox4x32_10(u32x4{(uint32_t)pos, 0u, (uint32_t)row, 2u}, slo, shi);
        const float u = ((float)(w[0] >> 9) + 0.5f) * 0x1.0p-23f;
        reject = !(u < expf(lp - lq));
      }
    }
    const uint32_t rej = (uint32_t)(__ballot(reject) >> (16 * sub)) & 0xffffu;
    if (rej && stop < 0) stop = c + __builtin_ctz(rej);
  }
  const bool bad_row = ((uint32_t)(__ballot(bad_any) >> (16 * sub)) & 0xffffu) != 0u;
  if (!live || p != 0) return;
  if (bad_row) status_or(status, DSPARK_STATUS_BAD_TOKEN);
  const int k = stop < 0 ? K : stop;
  n_acc[row] = k;
  pos_out[row] = k;
  if (greedy)
    next_token[row] = (int32_t)__float_as_uint(stats[((int64_t)row * (K + 1) + k) * kStat + 4]);
  else
    keys[row] = 0ull;  // the draw's key, folded by the resample pass's atomic maxima
}

// Gumbel-max draw at each row's stopping position: from max(0, p - q) when
// a draft was rejected there, from p at the position after the block.
__global__ __launch_bounds__(kThreads) void verify_resample_kernel(
    const float* __restrict__ draft, const float* __restrict__ target, const float* __restrict__ stats,
    const int32_t* __restrict__ pos_in, int K, int V, float invT, uint32_t slo, uint32_t shi, int vec,
    uint64_t* __restrict__ keys) {
  __shared__ uint64_t lds64[kThreads / 64];
  const int row = blockIdx.y, k = pos_in[row];
  const float* s = stats + ((int64_t)row * (K + 1) + k) * kStat;
  const float mt = s[0], ls_t = logf(s[1]), md = s[2], ls_d = k < K ? logf(s[3]) : 0.f;
  // p = exp(x invT - mt - ls_t) as 2^(x invT log2e - (mt + ls_t) log2e): one fma and one v_exp_f32
  const float cs = invT * kLog2eF, ot = (mt + ls_t) * kLog2eF, od = (md + ls_d) * kLog2eF;
  const float* t = target + ((int64_t)row * (K + 1) + k) * V;
  const float* d = draft + ((int64_t)row * K + (k < K ? k : 0)) * V;
  const int64_t nq = (V + 3) / 4;
  const int64_t q0 = (int64_t)blockIdx.x * nq / gridDim.x, q1 = (int64_t)(blockIdx.x + 1) * nq / gridDim.x;
  uint64_t best = 0;
  for (int64_t q = q0 + threadIdx.x; q < q1; q += kThreads) {
    // the quad's logits first (16-byte loads when rows are 16-byte aligned), then its noise
    f32x4 tv, dv = f32x4{0.f, 0.f, 0.f, 0.f};
    if (vec) {
      tv = *(const f32x4*)(t + 4 * q);
      if (k < K) dv = *(const f32x4*)(d + 4 * q);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t v = min(4 * q + e, (int64_t)V - 1);
        tv[e] = t[v];
        if (k < K) dv[e] = d[v];
      }
    }
    const u32x4 w = philox4x32_10(u32x4{(uint32_t)q, (uint32_t)k, (uint32_t)row, 1u}, slo, shi);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t v = 4 * q + e;
      if (v >= V) break;
      float z;
      if (k < K) {
        const float p = __builtin_amdgcn_exp2f(fmaf(tv[e], cs, -ot));
        const float qd = __builtin_amdgcn_exp2f(fmaf(dv[e], cs, -od));
        if (!(p > qd)) continue;
        z = kLn2F * __builtin_amdgcn_logf(p - qd) + gumbel_from_bits(w[e]);
      } else {
        z = tv[e] * invT + gumbel_from_bits(w[e]);
      }
      const uint64_t key = argmax_key(z, (uint32_t)v);
      best = key > best ? key : best;
    }
  }
  best = block_reduce(best, [](uint64_t a, uint64_t b) { return a > b ? a : b; }, lds64);
  if (threadIdx.x == 0 && best) atomicMax((unsigned long long*)&keys[row], (unsigned long long)best);
}

__global__ void verify_finalize_kernel(const uint64_t* __restrict__ keys, int32_t* __restrict__ next_token, int R,
                                       int V, int32_t* __restrict__ status) {
  const int row = blockIdx.x * blockDim.x + threadIdx.x;
  if (row >= R) return;
  uint32_t t = keys[row] ? argmax_key_index(keys[row]) : 0u;
  if (t >= (uint32_t)V) {
    status_or(status, DSPARK_STATUS_BAD_TOKEN);
    t = 0;
  }
  next_token[row] = (int32_t)t;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

extern "C" size_t dspark_verify_workspace_bytes(int R, int K) {
  if (R <= 0 || K < 0) return 0;
  return align256((size_t)R * (K + 1) * kStat * 4) + align256((size_t)R * 4) + align256((size_t)R * 8);
}

extern "C" int dspark_verify(const float* draft_logits, const float* target_logits, const int32_t* draft_tokens,
                             int32_t* n_accepted, int32_t* next_token, int R, int K, int V, float temperature,
                             uint64_t seed, void* ws, size_t ws_bytes, int32_t* dev_status, void* stream) {
  using namespace dspark_host;
  if (R < 0 || K < 0) return fail(DSPARK_ERR_INVALID_ARG, "verify: negative dimension");
  if (K > 1024) return fail(DSPARK_ERR_INVALID_ARG, "verify: K > 1024");
  if (V < 1) return fail(DSPARK_ERR_INVALID_ARG, "verify: V must be >= 1");
  if (!(temperature >= 0.f) || temperature == INFINITY)
    return fail(DSPARK_ERR_INVALID_ARG, "verify: temperature must be finite and >= 0");
  if (R == 0) return ok();
  if (!target_logits || !n_accepted || !next_token || (K > 0 && (!draft_logits || !draft_tokens)))
    return fail(DSPARK_ERR_INVALID_ARG, "verify: null required pointer");
  const size_t need = dspark_verify_workspace_bytes(R, K);
  if (!ws || ws_bytes < need) return fail(DSPARK_ERR_WORKSPACE, "verify: workspace %zu bytes < %zu", ws_bytes, need);
  if ((uintptr_t)ws % 256) return fail(DSPARK_ERR_INVALID_ARG, "verify: workspace not 256-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  float* stats = (float*)ws;
  int32_t* pos = (int32_t*)((char*)ws + align256((size_t)R * (K + 1) * kStat * 4));
  uint64_t* keys = (uint64_t*)((char*)pos + align256((size_t)R * 4));
  const int greedy = temperature == 0.f;
  const float invT = greedy ? 1.f : 1.f / temperature;
  const uint32_t slo = (uint32_t)seed, shi = (uint32_t)(seed >> 32);
  const int vec = V % 4 == 0 && (uintptr_t)target_logits % 16 == 0 && (uintptr_t)draft_logits % 16 == 0;
  hipLaunchKernelGGL(verify_stats_kernel, dim3(K + 1, R), dim3(kThreads), 0, s, draft_logits, target_logits, K, V,
                     invT, greedy, vec, stats);
  hipLaunchKernelGGL(verify_decide_kernel, dim3((R + 3) / 4), dim3(64), 0, s, draft_logits, target_logits,
                     draft_tokens, stats, R, K, V, invT, greedy, slo, shi, n_accepted, pos, next_token, dev_status,
                     keys);
  if (!greedy) {
    const int64_t nq = (V + 3) / 4;
    const int splits = (int)(nq < 64 * kThreads ? (nq + kThreads - 1) / kThreads : 64);
    hipLaunchKernelGGL(verify_resample_kernel, dim3(splits, R), dim3(kThreads), 0, s, draft_logits, target_logits,
                       stats, pos, K, V, invT, slo, shi, vec, keys);
    hipLaunchKernelGGL(verify_finalize_kernel, dim3((R + 255) / 256), dim3(256), 0, s, keys, next_token, R, V,
                       dev_status);
  }
  return check_launch("verify");
}
