// Gated and recurrent Markov heads (page 1, "03 · DSpark 建模", §3.7, the
// paper's Eq. 6 for the recurrent head; page 4, "DSpark 深度解读", §3.3, the
// table of head variants).
//
// Both heads replace the vanilla head's W1[x] (x the previous token) by a
// rank-r row E that also depends on the backbone hidden state h of the
// position; the bias is then E @ W2 as before:
//
//   gated:      E = sigmoid(W_g [h; W1[x]]) * W1[x]            W_g [r, d + r]
//   recurrent:  z = [s; W1[x]; h],  E = tanh(W_o z),
//               s <- sigmoid(W_g z) * s + (1 - sigmoid(W_g z)) * tanh(W_c z)
//               W_g, W_c, W_o [r, 2r + d], stacked [3, r, 2r + d]
//
// with the state s zero at the first position of each block and carried
// along the block (the next sampled token's position, or the next
// teacher-forced position).
//
// Work split:
// * The hidden-state part of every map, h @ W_h^T for all R x gamma
//   positions at once (it does not depend on the sampled tokens), is one
//   bf16 MFMA contraction over d: v_mfma_f32_16x16x32_bf16 with both
//   operands read straight from row-major memory as 16-byte pieces (lane
//   (n, g) of a fragment holds row n, entries 8g .. 8g+7 of the 32-wide
//   slab), 64 x 64 output tiles per workgroup of four waves.
// * Per position, a small kernel finishes the maps with the recurrent inputs
//   ([s; W1[x]], or W1[x] alone) in float32 (the state is never rounded),
//   applies the nonlinearities, writes E (float32) and the next state.
// * The step over the vocabulary is the vanilla head's kernel reading E from
//   that buffer (rounded to bf16 for the matrix cores) instead of W1[x].
#include "common.h"
#include "markov_step.h"

using namespace dspark;

namespace {

constexpr int kHeadGated = 1;
constexpr int kHeadRnn = 2;
constexpr int kProjTile = 64;   // output rows and columns per projection workgroup
constexpr int kRowsPer = 16;    // rows per recurrent-step workgroup
constexpr int kChanPer = 16;    // channels per recurrent-step workgroup
constexpr int kMaxRank = 512;

// P[i][c] = sum_k A[i][k] B[c][k] for i < M, c < N (bf16 in, float32 out).
// A rows are lda elements apart, B rows ldb; K, lda, ldb multiples of 8 and
// both bases 16-byte aligned (checked by the host).  Wave w of the
// workgroup owns rows 32(w & 1) .. +31 and columns 32(w >> 1) .. +31 of the
// tile: two A and two B fragments per 32-wide slab, four products.
__global__ __launch_bounds__(256) void head_proj_mfma(const uint16_t* __restrict__ A, int64_t lda,
                                                      const uint16_t* __restrict__ B, int64_t ldb,
                                                      float* __restrict__ P, int64_t ldp, int M, int N, int K) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int i0 = blockIdx.x * kProjTile + (wave & 1) * 32;
  const int c0 = blockIdx.y * kProjTile + (wave >> 1) * 32;
  const uint16_t* ap[2];
  const uint16_t* bp[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    ap[t] = A + (int64_t)min(i0 + 16 * t + n, M - 1) * lda;
    bp[t] = B + (int64_t)min(c0 + 16 * t + n, N - 1) * ldb;
  }
  f32x4 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  // two slabs per iteration, the next pair's pieces loaded before this
  // pair's products
  constexpr int U = 2;
  u32x4 fa[U][2], fb[U][2];
  auto load = [&](int k0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = k0 + 32 * u;
      const bool ok = k + 8 * g < K;  // K is a multiple of 8: the whole piece is in the row
      const int kc = ok ? k + 8 * g : 0;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const u32x4 x = *(const u32x4*)(ap[t] + kc), y = *(const u32x4*)(bp[t] + kc);
        fa[u][t] = ok ? x : u32x4{0u, 0u, 0u, 0u};
        fb[u][t] = ok ? y : u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  load(0);
  for (int k0 = 0; k0 < K; k0 += 32 * U) {
    u32x4 ca[U][2], cb[U][2];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int t = 0; t < 2; ++t) { ca[u][t] = fa[u][t]; cb[u][t] = fb[u][t]; }
    if (k0 + 32 * U < K) load(k0 + 32 * U);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = mfma16x16x32(cb[u][b], ca[u][a], acc[a][b]);
  }
  // lane (n, g) of product (a, b) holds row i0 + 16a + n, columns
  // c0 + 16b + 4g .. +3 (N is a multiple of 4)
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int i = i0 + 16 * a + n;
    if (i >= M) continue;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int c = c0 + 16 * b + 4 * g;
      if (c < N) *(f32x4*)(P + (int64_t)i * ldp + c) = acc[a][b];
    }
  }
}

template <bool kBf16>
__device__ __forceinline__ float ldw(const void* p, int64_t i) {
  return kBf16 ? __uint_as_float((uint32_t)((const uint16_t*)p)[i] << 16) : ((const float*)p)[i];
}

__device__ __forceinline__ float sigm(float x) { return 1.f / (1.f + expf(-x)); }

// One position of every row: rows row0 .. +15 and channels j0 .. +15 per
// workgroup, one (row, channel) per thread.
//   z = [s; W1[x]] (RNN, length 2r) or W1[x] (gated, length r), staged in LDS
//   acc_q = W_q,rec[j] . z  (q = gate, candidate, output; or the gate alone)
// W_q,rec rows are ldw elements apart, matrix q at wrec + q * mstride; the
// hidden-state part arrives in P[row, step, q * r + j].  The previous token
// is the caller's (prev_tok[row * prev_stride]) or the argmax folded in the
// previous step's keys.
template <bool RNN, bool kBf16W1>
__global__ __launch_bounds__(256) void head_step_kernel(
    const float* __restrict__ P, const void* __restrict__ w1, const uint16_t* __restrict__ wrec, int64_t ldwr,
    int64_t mstride, const int32_t* __restrict__ prev_tok, int64_t prev_stride,
    const uint64_t* __restrict__ keys_prev, const float* __restrict__ s_in, float* __restrict__ s_out,
    float* __restrict__ ebuf, int R, int gamma, int V, int r, int step, int32_t* __restrict__ status) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int zlen = RNN ? 2 * r : r;
  float* z = (float*)smem;                           // [kRowsPer][zlen]
  int* pv = (int*)(smem + (size_t)kRowsPer * zlen * 4);  // [kRowsPer]
  const int row0 = blockIdx.x * kRowsPer, j0 = blockIdx.y * kChanPer;
  if (threadIdx.x < kRowsPer) {
    const int row = row0 + threadIdx.x;
    int p = 0;
    if (row < R) {
      p = keys_prev ? (int)argmax_key_index(read_key(keys_prev, row, R)) : prev_tok[(int64_t)row * prev_stride];
      if (p < 0 || p >= V) {
        if (blockIdx.y == 0) status_or(status, DSPARK_STATUS_BAD_TOKEN);
        p = 0;
      }
    }
    pv[threadIdx.x] = p;
  }
  __syncthreads();
  for (int c = threadIdx.x; c < kRowsPer * zlen; c += 256) {
    const int rr = c / zlen, k = c % zlen, row = row0 + rr;
    float v = 0.f;
    if (row < R) {
      if (RNN && k < r) v = s_in[(int64_t)row * r + k];
      else v = ldw<kBf16W1>(w1, (int64_t)pv[rr] * r + (RNN ? k - r : k));
    }
    z[c] = v;
  }
  __syncthreads();
  const int i = threadIdx.x / kChanPer, j = j0 + threadIdx.x % kChanPer, row = row0 + i;
  constexpr int NQ = RNN ? 3 : 1;
  float acc[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) acc[q] = 0.f;
  const int jc = min(j, r - 1);
  const float* zr = z + i * zlen;
  for (int k = 0; k < zlen; k += 8) {
    const f32x4 z0 = *(const f32x4*)(zr + k), z1 = *(const f32x4*)(zr + k + 4);
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const u32x4 w = *(const u32x4*)(wrec + q * mstride + (int64_t)jc * ldwr + k);
      float a = acc[q];
      a = fmaf(bf16lo(w[0]), z0[0], a); a = fmaf(bf16hi(w[0]), z0[1], a);
      a = fmaf(bf16lo(w[1]), z0[2], a); a = fmaf(bf16hi(w[1]), z0[3], a);
      a = fmaf(bf16lo(w[2]), z1[0], a); a = fmaf(bf16hi(w[2]), z1[1], a);
      a = fmaf(bf16lo(w[3]), z1[2], a); a = fmaf(bf16hi(w[3]), z1[3], a);
      acc[q] = a;
    }
  }
  if (row >= R || j >= r) return;
  const int64_t pos = (int64_t)row * gamma + step;
  const float* p = P + pos * (NQ * r);
  if constexpr (RNN) {
    const float gt = sigm(acc[0] + p[j]);
    const float cand = tanhf(acc[1] + p[r + j]);
    ebuf[pos * r + j] = tanhf(acc[2] + p[2 * r + j]);
    s_out[(int64_t)row * r + j] = gt * zr[j] + (1.f - gt) * cand;
  } else {
    ebuf[pos * r + j] = sigm(acc[0] + p[j]) * zr[j];
  }
}

__global__ void fill_zero_f32(float* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Workspace layout: keys | P [R*gamma, NQ*r] | E [R*gamma, r] | s ping-pong [2, R, r]
struct Layout {
  size_t keys, proj, emb, state, total;
};
Layout layout(int kind, int R, int gamma, int r, int64_t nkeys) {
  const int nq = kind == kHeadRnn ? 3 : 1;
  Layout L;
  L.keys = 0;
  L.proj = align256((size_t)nkeys * 8);
  L.emb = L.proj + align256((size_t)R * gamma * nq * r * 4);
  L.state = L.emb + align256((size_t)R * gamma * r * 4);
  L.total = L.state + (kind == kHeadRnn ? align256((size_t)2 * R * r * 4) : 0);
  return L;
}

struct HeadArgs {
  int kind;
  const void* hidden;
  const void* w1;
  const void* whead;
  int wdtype;
  int R, gamma, V, r, d;
};

int check_head(const char* what, const HeadArgs& a) {
  using namespace dspark_host;
  if (a.kind != kHeadGated && a.kind != kHeadRnn) return fail(DSPARK_ERR_INVALID_ARG, "%s: unknown head kind %d", what, a.kind);
  if (a.R < 0 || a.gamma < 0) return fail(DSPARK_ERR_INVALID_ARG, "%s: negative dimension", what);
  if (a.gamma > 1024) return fail(DSPARK_ERR_INVALID_ARG, "%s: gamma > 1024", what);
  if (a.V < 1 || a.r < 8 || a.r > kMaxRank || a.r % 8)
    return fail(DSPARK_ERR_INVALID_ARG, "%s: need V >= 1 and r a multiple of 8 in [8, %d] (V=%d r=%d)", what,
                kMaxRank, a.V, a.r);
  if (a.d < 8 || a.d % 8) return fail(DSPARK_ERR_INVALID_ARG, "%s: d must be a positive multiple of 8 (got %d)", what, a.d);
  if (a.wdtype != DSPARK_BF16 && a.wdtype != DSPARK_F32)
    return fail(DSPARK_ERR_INVALID_ARG, "%s: unknown wdtype %d", what, a.wdtype);
  return 0;
}

// The hidden-state projection for all positions, then per position the
// recurrent kernel and (through `per_step`) the vocabulary step.
template <typename PerStep>
hipError_t run_head(const HeadArgs& a, const int32_t* prev_tok, int64_t prev_stride, int prev_step_stride,
                    const uint64_t* (*keys_prev_of)(void*, int), void* keys_ctx, char* ws, const Layout& L,
                    int32_t* status, hipStream_t s, PerStep per_step) {
  const bool rnn = a.kind == kHeadRnn;
  const int nq = rnn ? 3 : 1;
  const int64_t ldw = rnn ? 2 * (int64_t)a.r + a.d : (int64_t)a.d + a.r;
  const uint16_t* wh = (const uint16_t*)a.whead;
  float* P = (float*)(ws + L.proj);
  float* E = (float*)(ws + L.emb);
  float* S = (float*)(ws + L.state);
  const int M = a.R * a.gamma, N = nq * a.r;
  // h-part columns: gated [h; e] -> column 0; recurrent [s; e; h] -> column 2r.
  // The stacked recurrent maps are one [3r, 2r + d] matrix.
  const uint16_t* Bh = wh + (rnn ? 2 * a.r : 0);
  hipLaunchKernelGGL(head_proj_mfma, dim3((M + kProjTile - 1) / kProjTile, (N + kProjTile - 1) / kProjTile),
                     dim3(256), 0, s, (const uint16_t*)a.hidden, (int64_t)a.d, Bh, ldw, P, (int64_t)N, M, N, a.d);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (rnn) {
    const int64_t n = (int64_t)a.R * a.r;  // s_0 = 0
    hipLaunchKernelGGL(fill_zero_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, S, n);
  }
  const uint16_t* wrec = wh + (rnn ? 0 : a.d);
  const int64_t mstride = (int64_t)a.r * ldw;
  const size_t shm = (size_t)kRowsPer * (rnn ? 2 : 1) * a.r * 4 + kRowsPer * 4;
  const dim3 grid((a.R + kRowsPer - 1) / kRowsPer, (a.r + kChanPer - 1) / kChanPer);
  for (int k = 0; k < a.gamma; ++k) {
    const float* sin = S + (int64_t)(k & 1) * a.R * a.r;
    float* sout = S + (int64_t)((k + 1) & 1) * a.R * a.r;
    const uint64_t* kp = keys_prev_of ? keys_prev_of(keys_ctx, k) : nullptr;
    const int32_t* pt = prev_tok ? prev_tok + (int64_t)k * prev_step_stride : nullptr;
#define DSPARK_HS_LAUNCH(RN, WB)                                                                              \
  if (shm > 65536 && k == 0)                                                                                  \
    (void)hipFuncSetAttribute((const void*)head_step_kernel<RN, WB>,                                          \
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);                          \
  hipLaunchKernelGGL((head_step_kernel<RN, WB>), grid, dim3(256), shm, s, P, a.w1, wrec, ldw, mstride, pt,     \
                     prev_stride, kp, sin, sout, E, a.R, a.gamma, a.V, a.r, k, status)
    if (rnn) {
      if (a.wdtype == DSPARK_BF16) { DSPARK_HS_LAUNCH(true, true); }
      else { DSPARK_HS_LAUNCH(true, false); }
    } else {
      if (a.wdtype == DSPARK_BF16) { DSPARK_HS_LAUNCH(false, true); }
      else { DSPARK_HS_LAUNCH(false, false); }
    }
#undef DSPARK_HS_LAUNCH
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = per_step(k, E)) != hipSuccess) return e;
  }
  return hipSuccess;
}

int check_alignment(const char* what, const HeadArgs& a) {
  using namespace dspark_host;
  if ((uintptr_t)a.hidden % 16 || (uintptr_t)a.whead % 16)
    return fail(DSPARK_ERR_INVALID_ARG, "%s: hidden and head weights must be 16-byte aligned", what);
  return 0;
}

struct SampleKeys {
  uint64_t* keys;
  int64_t per_step;
};
const uint64_t* sample_keys_prev(void* ctx, int k) {
  const SampleKeys* c = (const SampleKeys*)ctx;
  return k == 0 ? nullptr : c->keys + (int64_t)(k - 1) * c->per_step;
}

}  // namespace

extern "C" size_t dspark_markov_head_sample_workspace_bytes(int kind, int R, int gamma, int V, int r) {
  (void)V;
  if (R <= 0 || gamma <= 0 || r <= 0 || (kind != kHeadGated && kind != kHeadRnn)) return 0;
  return layout(kind, R, gamma, r, (int64_t)gamma * keys_per_step(R)).total;
}

extern "C" int dspark_markov_head_sample(int kind, const float* base_logits, const void* hidden, const void* w1,
                                        const void* w2, const void* whead, const int32_t* first_prev,
                                        int32_t* tokens, float* step_logits, int R, int gamma, int V, int r, int d,
                                        int wdtype, float temperature, uint64_t seed, void* ws, size_t ws_bytes,
                                        int32_t* dev_status, void* stream) {
  using namespace dspark_host;
  const HeadArgs a{kind, hidden, w1, whead, wdtype, R, gamma, V, r, d};
  if (int rc = check_head("markov_head_sample", a)) return rc;
  if (!(temperature >= 0.f) || temperature == INFINITY)
    return fail(DSPARK_ERR_INVALID_ARG, "markov_head_sample: temperature must be finite and >= 0");
  if ((int64_t)R * gamma == 0) return ok();
  if (!base_logits || !hidden || !w1 || !w2 || !whead || !first_prev || !tokens)
    return fail(DSPARK_ERR_INVALID_ARG, "markov_head_sample: null required pointer");
  if (int rc = check_alignment("markov_head_sample", a)) return rc;
  const size_t need = dspark_markov_head_sample_workspace_bytes(kind, R, gamma, V, r);
  if (!ws || ws_bytes < need)
    return fail(DSPARK_ERR_WORKSPACE, "markov_head_sample: workspace %zu bytes < %zu", ws_bytes, need);
  if ((uintptr_t)ws % 256) return fail(DSPARK_ERR_INVALID_ARG, "markov_head_sample: workspace not 256-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  const Layout L = layout(kind, R, gamma, r, (int64_t)gamma * keys_per_step(R));
  SampleKeys sk{(uint64_t*)ws, keys_per_step(R)};
  hipError_t e = markov_zero_keys(sk.keys, (int64_t)gamma * sk.per_step, s);
  if (e == hipSuccess)
    e = run_head(a, first_prev, 1, 0, sample_keys_prev, &sk, (char*)ws, L, dev_status, s,
                 [&](int k, const float* E) {
                   return markov_step_embedded(base_logits, E, w2, wdtype, sk.keys + (int64_t)k * sk.per_step,
                                               step_logits, R, gamma, V, r, k, 0.f, temperature, seed, s);
                 });
  if (e == hipSuccess) e = markov_finalize_tokens(sk.keys, tokens, R, gamma, V, dev_status, s);
  if (e != hipSuccess) return fail(DSPARK_ERR_HIP, "markov_head_sample: %s", hipGetErrorString(e));
  return check_launch("markov_head_sample");
}

extern "C" size_t dspark_markov_head_block_logits_workspace_bytes(int kind, int B, int gamma, int V, int r) {
  (void)V;
  if (B <= 0 || gamma <= 0 || r <= 0 || (kind != kHeadGated && kind != kHeadRnn)) return 0;
  return layout(kind, B, gamma, r, keys_per_step(B * gamma)).total;
}

extern "C" int dspark_markov_head_block_logits(int kind, const float* base_logits, const void* hidden,
                                              const void* w1, const void* w2, const void* whead,
                                              const int32_t* prev, float* logits, int32_t* argmax_tokens, int B,
                                              int gamma, int V, int r, int d, int wdtype, float softcap, void* ws,
                                              size_t ws_bytes, int32_t* dev_status, void* stream) {
  using namespace dspark_host;
  const HeadArgs a{kind, hidden, w1, whead, wdtype, B, gamma, V, r, d};
  if (int rc = check_head("markov_head_block_logits", a)) return rc;
  if (!(softcap >= 0.f) || softcap == INFINITY)
    return fail(DSPARK_ERR_INVALID_ARG, "markov_head_block_logits: softcap must be finite and >= 0");
  if ((int64_t)B * gamma == 0) return ok();
  if ((int64_t)B * gamma > (1 << 30)) return fail(DSPARK_ERR_INVALID_ARG, "markov_head_block_logits: too many rows");
  if (!base_logits || !hidden || !w1 || !w2 || !whead || !prev || !logits)
    return fail(DSPARK_ERR_INVALID_ARG, "markov_head_block_logits: null required pointer");
  if (int rc = check_alignment("markov_head_block_logits", a)) return rc;
  const size_t need = dspark_markov_head_block_logits_workspace_bytes(kind, B, gamma, V, r);
  if (!ws || ws_bytes < need)
    return fail(DSPARK_ERR_WORKSPACE, "markov_head_block_logits: workspace %zu bytes < %zu", ws_bytes, need);
  if ((uintptr_t)ws % 256)
    return fail(DSPARK_ERR_INVALID_ARG, "markov_head_block_logits: workspace not 256-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  const int N = B * gamma;
  const Layout L = layout(kind, B, gamma, r, keys_per_step(N));
  uint64_t* keys = (uint64_t*)ws;
  hipError_t e = markov_zero_keys(keys, keys_per_step(N), s);
  // teacher forcing: position k of block b takes prev[b * gamma + k]; the
  // recurrent state runs along the block; all E rows first, then one
  // vocabulary pass over the N rows
  if (e == hipSuccess)
    e = run_head(a, prev, gamma, 1, nullptr, nullptr, (char*)ws, L, dev_status, s,
                 [](int, const float*) { return hipSuccess; });
  if (e == hipSuccess)
    e = markov_step_embedded(base_logits, (const float*)((char*)ws + L.emb), w2, wdtype, keys, logits, N, 1, V, r,
                             0, softcap, 0.f, 0, s);
  if (e == hipSuccess && argmax_tokens) e = markov_finalize_tokens(keys, argmax_tokens, N, 1, V, dev_status, s);
  if (e != hipSuccess) return fail(DSPARK_ERR_HIP, "markov_head_block_logits: %s", hipGetErrorString(e));
  return check_launch("markov_head_block_logits");
}
