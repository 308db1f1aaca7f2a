// Cumulative-product eval mask (page 1, "03 · DSpark 建模", §3.1 and §3.6).
//
// One thread per block (b, a) walks the gamma positions, ANDs the three
// per-position conditions (kept block, label inside the sequence, label
// supervised by the loss mask) and keeps the running product, so the output
// is the contiguous valid prefix.  Integer work only; the whole op is a few
// kilobytes and is bound by launch latency.
#include "common.h"

namespace {

__global__ __launch_bounds__(256) void eval_mask_kernel(
    const int32_t* __restrict__ anchor, const uint8_t* __restrict__ keep,
    const int32_t* __restrict__ seq_lens, const uint8_t* __restrict__ loss_mask,
    uint8_t* __restrict__ out, int B, int A, int gamma, int S_stride, int32_t* status) {
  const int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (blk >= (int64_t)B * A) return;
  const int b = (int)(blk / A);
  const int32_t p = anchor[blk];
  if (keep[blk] != 0 && p < 0) dspark::status_or(status, DSPARK_STATUS_BAD_ANCHOR);
  const bool kept = keep[blk] != 0 && p >= 0;
  const int32_t len = seq_lens[b];
  const uint8_t* lm = loss_mask ? loss_mask + (int64_t)b * S_stride : nullptr;
  uint8_t* o = out + blk * gamma;
  int running = kept ? 1 : 0;
  for (int k = 0; k < gamma; ++k) {
    if (running) {
      const int64_t L = (int64_t)p + 1 + k;
      bool valid = L < len;
      if (valid && lm) {
        if (L >= S_stride) {
          dspark::status_or(status, DSPARK_STATUS_BAD_LABEL);
          valid = false;
        } else {
          valid = lm[L] != 0;
        }
      }
      running = valid ? 1 : 0;
    }
    o[k] = (uint8_t)running;
  }
}

}  // namespace

extern "C" int dspark_eval_mask(const int32_t* anchor_pos, const uint8_t* keep_mask,
                                const int32_t* seq_lens, const uint8_t* loss_mask,
                                uint8_t* eval_mask, int B, int A, int gamma, int S_stride,
                                int32_t* dev_status, void* stream) {
  using namespace dspark_host;
  if (B < 0 || A < 0 || gamma < 0)
    return fail(DSPARK_ERR_INVALID_ARG, "eval_mask: negative dimension (B=%d A=%d gamma=%d)", B, A, gamma);
  if ((int64_t)B * A * gamma == 0) return ok();
  if (!anchor_pos || !keep_mask || !seq_lens || !eval_mask)
    return fail(DSPARK_ERR_INVALID_ARG, "eval_mask: null required pointer");
  if (loss_mask && S_stride <= 0)
    return fail(DSPARK_ERR_INVALID_ARG, "eval_mask: S_stride must be > 0 with a loss mask");
  const int64_t n = (int64_t)B * A;
  const int threads = 256;
  const int64_t grid = (n + threads - 1) / threads;
  if (grid > 0x7fffffff) return fail(DSPARK_ERR_INVALID_ARG, "eval_mask: too many blocks");
  hipLaunchKernelGGL(eval_mask_kernel, dim3((unsigned)grid), dim3(threads), 0,
                     (hipStream_t)stream, anchor_pos, keep_mask, seq_lens, loss_mask, eval_mask,
                     B, A, gamma, S_stride, dev_status);
  return check_launch("eval_mask");
}
