// Confidence head, prefix survival and the hardware-aware verify-length
// scheduler (page 1, "03 · DSpark 建模", §3.8; page 4, "DSpark 深度解读",
// §3.4 and §5.1).
//
// For draft row n (position k = 1 .. gamma of its block):
//
//   c_n = sigmoid(w_h . h_n + w_e . W1[prev_n] + b)       (w_e term optional)
//   a_k = prod_{i <= k} c_i                                (prefix survival)
//   Theta_l = (1 + sum_{k <= l} a_k) * SPS[l],  l = 0 .. gamma
//   verify length = the last l before Theta first drops    (causal greedy)
//
// One workgroup of 16 waves per block: its waves take the block's rows in
// turn (a dot product over the hidden state with 16-byte loads when the row
// length allows, plus the previous token's Markov embedding, reduced across
// the wave), then one thread runs the block's prefix product and the
// early-stopping scan.  The work is a few tens of MB at serving sizes.
#include "common.h"

using namespace dspark;

namespace {

constexpr int kThreads = 1024;  // one wave per block position up to gamma = 16
constexpr int kMaxGamma = 1024;

template <bool kBf16>
__device__ __forceinline__ float ld(const void* p, int64_t i) {
  return kBf16 ? __uint_as_float((uint32_t)((const uint16_t*)p)[i] << 16) : ((const float*)p)[i];
}

// dot(hidden row, w_h) of one wave: 16-byte loads (8 bf16 or 4 fp32 values
// per lane and step) when VEC, else one element per lane and step.
template <bool kBf16, bool VEC>
__device__ __forceinline__ float row_dot(const void* hidden, int64_t row, int H, const float* wh, int lane) {
  float acc = 0.f;
  if constexpr (VEC) {
    constexpr int kEl = kBf16 ? 8 : 4;
    const u32x4* hp = (const u32x4*)((const char*)hidden + row * (int64_t)H * (kBf16 ? 2 : 4));
    const f32x4* wp = (const f32x4*)wh;
    for (int c = lane; c < H / kEl; c += 64) {
      const u32x4 x = hp[c];
      if constexpr (kBf16) {
        const f32x4 w0 = wp[2 * c], w1 = wp[2 * c + 1];
        acc = fmaf(bf16lo(x[0]), w0[0], acc); acc = fmaf(bf16hi(x[0]), w0[1], acc);
        acc = fmaf(bf16lo(x[1]), w0[2], acc); acc = fmaf(bf16hi(x[1]), w0[3], acc);
        acc = fmaf(bf16lo(x[2]), w1[0], acc); acc = fmaf(bf16hi(x[2]), w1[1], acc);
        acc = fmaf(bf16lo(x[3]), w1[2], acc); acc = fmaf(bf16hi(x[3]), w1[3], acc);
      } else {
        const f32x4 w0 = wp[c];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = fmaf(__uint_as_float(x[e]), w0[e], acc);
      }
    }
  } else {
    for (int j = lane; j < H; j += 64) acc = fmaf(ld<kBf16>(hidden, row * H + j), wh[j], acc);
  }
  return acc;
}

template <bool kBf16H, bool kBf16W, bool VEC>
__global__ __launch_bounds__(kThreads) void confidence_schedule_kernel(
    const void* __restrict__ hidden, const float* __restrict__ wh, float bias, const void* __restrict__ w1,
    const int32_t* __restrict__ prev, const float* __restrict__ we, int r, int V, const float* __restrict__ sps,
    float* __restrict__ conf, float* __restrict__ surv, int32_t* __restrict__ vlen, float* __restrict__ theta,
    int64_t nblocks, int gamma, int H, int32_t* __restrict__ status) {
  __shared__ float cbuf[kMaxGamma];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = kThreads / 64;
  for (int64_t blk = blockIdx.x; blk < nblocks; blk += gridDim.x) {
    for (int k = w; k < gamma; k += nw) {
      const int64_t row = blk * gamma + k;
      float acc = row_dot<kBf16H, VEC>(hidden, row, H, wh, lane);
      if (we) {
        int p = prev[row];
        if (p < 0 || p >= V) {
          if (lane == 0) status_or(status, DSPARK_STATUS_BAD_TOKEN);
          p = 0;
        }
        for (int j = lane; j < r; j += 64) acc = fmaf(ld<kBf16W>(w1, (int64_t)p * r + j), we[j], acc);
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, kWave);
      if (lane == 0) {
        const float c = 1.f / (1.f + expf(-(acc + bias)));
        cbuf[k] = c;
        if (conf) conf[row] = c;
      }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      float a = 1.f, sum = 1.f, prev_th = sps[0];
      int l = 0;
      bool stopped = false;
      if (theta) theta[blk * (gamma + 1)] = prev_th;
      for (int k = 1; k <= gamma; ++k) {
        a *= cbuf[k - 1];
        sum += a;
        if (surv) surv[blk * gamma + k - 1] = a;
        const float th = sum * sps[k];
        if (theta) theta[blk * (gamma + 1) + k] = th;
        if (!stopped) {
          if (th < prev_th) stopped = true;
          else l = k;
          prev_th = th;
        }
      }
      vlen[blk] = l;
    }
    __syncthreads();  // cbuf is reused by the next block
  }
}

}  // namespace

extern "C" int dspark_confidence_schedule(const void* hidden, int hdtype, const float* weight_h, float bias,
                                          const void* w1, int wdtype, const int32_t* prev, const float* weight_e,
                                          int r, int V, const float* sps, float* confidence, float* survival,
                                          int32_t* verify_len, float* theta, int B, int A, int gamma, int H,
                                          int32_t* dev_status, void* stream) {
  using namespace dspark_host;
  if (B < 0 || A < 0 || gamma < 0) return fail(DSPARK_ERR_INVALID_ARG, "confidence_schedule: negative dimension");
  if (gamma > kMaxGamma) return fail(DSPARK_ERR_INVALID_ARG, "confidence_schedule: gamma > %d", kMaxGamma);
  if (H < 1) return fail(DSPARK_ERR_INVALID_ARG, "confidence_schedule: H must be >= 1 (got %d)", H);
  if (hdtype != DSPARK_BF16 && hdtype != DSPARK_F32)
    return fail(DSPARK_ERR_INVALID_ARG, "confidence_schedule: unknown hidden dtype %d", hdtype);
  const bool markov = weight_e != nullptr;
  if (markov) {
    if (!w1 || !prev) return fail(DSPARK_ERR_INVALID_ARG, "confidence_schedule: Markov input needs w1 and prev");
    if (r < 1 || V < 1) return fail(DSPARK_ERR_INVALID_ARG, "confidence_schedule: need r >= 1 and V >= 1");
    if (wdtype != DSPARK_BF16 && wdtype != DSPARK_F32)
      return fail(DSPARK_ERR_INVALID_ARG, "confidence_schedule: unknown w1 dtype %d", wdtype);
  }
  if (!(bias == bias) || bias == INFINITY || bias == -INFINITY)
    return fail(DSPARK_ERR_INVALID_ARG, "confidence_schedule: bias must be finite");
  const int64_t nblocks = (int64_t)B * A;
  if (nblocks == 0 || gamma == 0) return ok();
  if (!hidden || !weight_h || !sps || !verify_len)
    return fail(DSPARK_ERR_INVALID_ARG, "confidence_schedule: null required pointer");
  hipStream_t s = (hipStream_t)stream;
  const unsigned grid = (unsigned)(nblocks < 4096 ? nblocks : 4096);
  const bool hb = hdtype == DSPARK_BF16, wb = !markov || wdtype == DSPARK_BF16;
  const bool vec = H % (hb ? 8 : 4) == 0 && (uintptr_t)hidden % 16 == 0 && (uintptr_t)weight_h % 16 == 0;
#define DSPARK_CS_LAUNCH(HB, WB, VC)                                                                           \
  hipLaunchKernelGGL((confidence_schedule_kernel<HB, WB, VC>), dim3(grid), dim3(kThreads), 0, s, hidden,      \
                     weight_h, bias, w1, prev, weight_e, r, V, sps, confidence, survival, verify_len, theta,  \
                     nblocks, gamma, H, dev_status)
  if (vec) {
    if (hb && wb) DSPARK_CS_LAUNCH(true, true, true);
    else if (hb) DSPARK_CS_LAUNCH(true, false, true);
    else if (wb) DSPARK_CS_LAUNCH(false, true, true);
    else DSPARK_CS_LAUNCH(false, false, true);
  } else {
    if (hb && wb) DSPARK_CS_LAUNCH(true, true, false);
    else if (hb) DSPARK_CS_LAUNCH(true, false, false);
    else if (wb) DSPARK_CS_LAUNCH(false, true, false);
    else DSPARK_CS_LAUNCH(false, false, false);
  }
#undef DSPARK_CS_LAUNCH
  return check_launch("confidence_schedule");
}
