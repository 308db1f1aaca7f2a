// Block-masked dual-source attention (page 1, "03 · DSpark 建模", §3.4 block
// attention mask and §3.5 custom attention; page 4, "DSpark 深度解读", §3.2).
//
// Queries come from the draft blocks only; keys/values are the context
// projections followed by each block's own projections.  A block sees the
// context strictly before its anchor plus its own gamma keys; a keep=0 block
// is fully masked (zeros, lse = -inf).  No mask is ever materialised: the
// rules are evaluated per score inside the kernel.
//
// gfx950 design (bf16 in, fp32 accumulate):
// * Row space.  For request b and key/value head kvh the query rows of all
//   blocks and of the Hq/Hkv query heads sharing kvh are laid out as
//   u = (a * group + hg) * gamma + k and cut into 64-row tiles, so one tile
//   packs several heads (and, for short blocks, several consecutive blocks)
//   against the same keys: the MFMA M/N extent is filled by GQA packing, not
//   by padding gamma.
// * Work item = (b, kvh, tile, context chunk of kChunk keys).  A tile's
//   context length is the largest anchor of its kept blocks; chunks past it
//   exit at once, so block-sparse work is skipped at chunk granularity and
//   masked per score inside the last slab.  The own-block keys of the tile's
//   blocks form extra 32-key slabs of chunk 0 with a block-diagonal mask.
// * Four waves per workgroup: two 32-row groups x two key parities.  Per
//   32-key slab a wave computes S^T = K Q^T (v_mfma_f32_32x32x16_bf16; K rows
//   and Q rows are loaded as 16-byte row pieces), so each lane owns ONE query
//   row: the online-softmax max, sum and rescale are lane-local plus a single
//   cross-half exchange.  The probabilities feed O^T = V^T P^T straight from
//   the S^T accumulator layout (no transpose of P); V's head dimension is
//   permuted (slot m of product j is d = NJ*m + j) so every lane loads
//   NJ*2-byte pieces of key rows and transposes them in registers.
// * Parities merge through LDS; chunks of one tile merge through workspace
//   partials folded by the last chunk to finish (fixed order: deterministic).
// * Workgroup ids run kvh fastest, so with 8 KV heads the eight XCDs each
//   serve one head and keep its context K/V in their own L2.
#include "common.h"

using namespace dspark;

namespace {

constexpr int kThreads = 256;
constexpr int kTileRows = 64;
constexpr int kChunk = 1024;  // context keys per work item
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;

struct Params {
  const uint16_t* q;
  const uint16_t* kc;
  const uint16_t* vc;
  const int32_t* offs;
  const uint16_t* kb;
  const uint16_t* vb;
  const int32_t* anchor;
  const uint8_t* keep;
  uint16_t* out;
  float* lse;
  float* partial;     // [items][kTileRows][D + 2]
  unsigned* counter;  // [ntiles * B * Hkv]
  int32_t* status;
  int B, A, gamma, Hq, Hkv, group, ntiles, nrows;  // nrows = A * group * gamma
  int total_ctx, max_ctx;
  float scale;
};

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// Context extent of request b, clamped into the K/V allocation.
__device__ __forceinline__ void ctx_range(const Params& p, int b, int& c0, int& S, bool flag) {
  int o0 = p.offs[b], o1 = p.offs[b + 1];
  const int s0 = clampi(o0, 0, p.total_ctx), s1 = clampi(o1, s0, p.total_ctx);
  int len = s1 - s0;
  if (len > p.max_ctx) len = p.max_ctx;
  if (flag && (s0 != o0 || s1 != o1 || len != o1 - o0)) status_or(p.status, DSPARK_STATUS_BAD_OFFSETS);
  c0 = s0;
  S = len;
}

__device__ __forceinline__ int visible_ctx(const Params& p, int b, int a, int S, bool flag) {
  if (!p.keep[(int64_t)b * p.A + a]) return -1;  // masked block
  const int an = p.anchor[(int64_t)b * p.A + a];
  if (flag && (an < 0 || an > S)) status_or(p.status, DSPARK_STATUS_BAD_ANCHOR);
  return clampi(an, 0, S);
}

template <int D>
__global__ __launch_bounds__(kThreads) void block_attn_mfma(Params p) {
  constexpr int NJ = D / 32;  // head-dim groups of the PV product
  constexpr int KK = D / 16;  // k-steps of the QK product
  __shared__ float mrg[2][D + 2][32];
  __shared__ int s_last;

  // ---- decode the work item (kvh fastest)
  int wid = blockIdx.x;
  const int kvh = wid % p.Hkv; wid /= p.Hkv;
  const int b = wid % p.B; wid /= p.B;
  const int tile = wid % p.ntiles;
  const int chunk = wid / p.ntiles;
  int c0, S;
  ctx_range(p, b, c0, S, chunk == 0 && tile == 0 && kvh == 0 && threadIdx.x == 0);
  const int rpb = p.group * p.gamma;  // rows per block
  const int u0 = tile * kTileRows;
  const int a_lo = u0 / rpb;
  const int a_hi = min(p.A - 1, (u0 + kTileRows - 1) / rpb);
  int L = 0;
  bool any_kept = false;
  for (int a = a_lo; a <= a_hi; ++a) {
    const int v = visible_ctx(p, b, a, S, false);
    if (v >= 0) { any_kept = true; L = max(L, v); }
  }
  const int nch = L > 0 ? (L + kChunk - 1) / kChunk : 1;
  if (chunk >= nch) return;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rg = wave & 1, par = wave >> 1;
  const int h = lane >> 5, r32 = lane & 31;
  // this lane's query row
  const int u = u0 + rg * 32 + r32;
  const bool row_ok = u < p.nrows;
  const int ua = row_ok ? u / rpb : a_lo;
  const int uhg = (u / p.gamma) % p.group, uk = u % p.gamma;
  const int qh = kvh * p.group + uhg;
  int lim = row_ok ? visible_ctx(p, b, ua, S, chunk == 0 && par == 0 && h == 0) : -1;
  const bool kept = lim >= 0;
  if (!kept) lim = 0;
  const int64_t qrow = ((int64_t)b * p.A * p.gamma + (int64_t)ua * p.gamma + uk) * p.Hq + qh;

  // Q^T operand pieces: d = 16*kk + 8*h .. +7
  u32x4 qf[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk)
    qf[kk] = row_ok ? *(const u32x4*)(p.q + qrow * D + kk * 16 + h * 8) : u32x4{0u, 0u, 0u, 0u};

  const int cbeg = chunk * kChunk, cend = min(L, cbeg + kChunk);
  const int n_ctx_slabs = (cend - cbeg + 31) / 32;
  const int n_own = (a_hi - a_lo + 1) * p.gamma;
  const int n_own_slabs = (chunk == 0 && any_kept) ? (n_own + 31) / 32 : 0;
  const int nslab = n_ctx_slabs + n_own_slabs;
  const float c = p.scale * kLog2e;

  float m = -INFINITY, l = 0.f;
  f32x16 o[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[j][r] = 0.f;

  const int64_t kv_stride = (int64_t)p.Hkv * D;  // elements between consecutive keys
  for (int s = par; s < nslab; s += 2) {
    const bool own = s >= n_ctx_slabs;
    // -- key rows this lane loads: K as the A operand (key slot r32) and the
    //    V pieces for the 16 keys of its half (slots 8q + 4h + i)
    const uint16_t *kbase, *vbase;
    int64_t krow;
    int j0 = 0, os = 0;
    if (!own) {
      j0 = cbeg + s * 32;
      krow = (int64_t)c0 + min(j0 + r32, S - 1);
      kbase = p.kc; vbase = p.vc;
    } else {
      os = (s - n_ctx_slabs) * 32;
      const int o_i = min(os + r32, n_own - 1);
      krow = (int64_t)b * p.A * p.gamma + (int64_t)a_lo * p.gamma + o_i;
      kbase = p.kb; vbase = p.vb;
    }
    u32x4 kf[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      kf[kk] = *(const u32x4*)(kbase + (krow * p.Hkv + kvh) * D + kk * 16 + h * 8);
    // V pieces: key of (t, s8) is 8*(2t + s8/4) + 4h + s8%4, head dims NJ*r32 .. +NJ-1
    uint32_t vraw[2][8][NJ / 2 > 0 ? NJ / 2 : 1];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int s8 = 0; s8 < 8; ++s8) {
        const int ks = 8 * (2 * t + s8 / 4) + 4 * h + (s8 & 3);
        int64_t vrow;
        if (!own) vrow = (int64_t)c0 + min(j0 + ks, S - 1);
        else vrow = (int64_t)b * p.A * p.gamma + (int64_t)a_lo * p.gamma + min(os + ks, n_own - 1);
        const uint16_t* vp = vbase + (vrow * p.Hkv + kvh) * D + NJ * r32;
        if constexpr (NJ == 4) {
          const u32x2 w = *(const u32x2*)vp;
          vraw[t][s8][0] = w.x;
          vraw[t][s8][1] = w.y;
        } else {
          vraw[t][s8][0] = *(const uint32_t*)vp;
        }
      }
    // -- S^T = K Q^T: lane holds row r32, keys 8*(i/4) + 4h + i%4
    f32x16 sc;
#pragma unroll
    for (int i = 0; i < 16; ++i) sc[i] = 0.f;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) sc = mfma32x32x16(kf[kk], qf[kk], sc);
    // -- mask and online softmax (lane-local row)
    float smax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int ks = 8 * (i / 4) + 4 * h + (i & 3);
      bool vis;
      if (!own) {
        const int j = j0 + ks;
        vis = kept && j < cend && j < lim;
      } else {
        const int o_i = os + ks;
        vis = kept && o_i < n_own && (a_lo + o_i / p.gamma) == ua;
      }
      sc[i] = vis ? sc[i] : -INFINITY;
      smax = fmaxf(smax, sc[i]);
    }
    smax = fmaxf(smax, __shfl_xor(smax, 32, kWave));
    const float mnew = fmaxf(m, smax);
    const float muse = mnew == -INFINITY ? 0.f : mnew;
    const float alpha = __builtin_amdgcn_exp2f((m - muse) * c);
    float psum = 0.f;
    u32x4 pb[2];
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[i], c, -muse * c));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[i + 1], c, -muse * c));
      psum += p0 + p1;
      pb[i / 8][(i % 8) / 2] = f32_to_bf16(p0) | (f32_to_bf16(p1) << 16);
    }
    psum += __shfl_xor(psum, 32, kWave);
    l = l * alpha + psum;
    m = mnew;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[j][r] *= alpha;
    // -- O^T += V^T P^T, two 16-key halves
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        u32x4 va;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t lo = vraw[t][2 * w][j / 2], hi = vraw[t][2 * w + 1][j / 2];
          va[w] = (j & 1) ? pack_hi(lo, hi) : pack_lo(lo, hi);
        }
        o[j] = mfma32x32x16(va, pb[t], o[j]);
      }
    }
  }

  // ---- merge the two key parities of each row group through LDS
  if (par == 1) {
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int d = NJ * (8 * (r / 4) + 4 * h + (r & 3)) + j;
        mrg[rg][d][r32] = o[j][r];
      }
    if (h == 0) { mrg[rg][D][r32] = m; mrg[rg][D + 1][r32] = l; }
  }
  __syncthreads();
  if (par == 0) {
    const float m1 = mrg[rg][D][r32], l1 = mrg[rg][D + 1][r32];
    const float mn = fmaxf(m, m1);
    const float mu = mn == -INFINITY ? 0.f : mn;
    const float a0 = __builtin_amdgcn_exp2f((m - mu) * c), a1 = __builtin_amdgcn_exp2f((m1 - mu) * c);
    l = l * a0 + l1 * a1;
    m = mn;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int d = NJ * (8 * (r / 4) + 4 * h + (r & 3)) + j;
        o[j][r] = o[j][r] * a0 + mrg[rg][d][r32] * a1;
      }
  }

  // ---- several chunks: publish the partial, the last chunk folds them all
  const int tile_id = (tile * p.B + b) * p.Hkv + kvh;
  if (nch > 1) {
    const int64_t item = ((int64_t)chunk * p.ntiles * p.B + (int64_t)tile * p.B + b) * p.Hkv + kvh;
    float* part = p.partial + item * kTileRows * (D + 2);
    if (par == 0) {
      float* pr = part + (rg * 32 + r32) * (D + 2);
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) pr[NJ * (8 * (r / 4) + 4 * h + (r & 3)) + j] = o[j][r];
      if (h == 0) { pr[D] = m; pr[D + 1] = l; }
    }
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
      const unsigned old = atomicAdd(p.counter + tile_id, 1u);
      s_last = old == (unsigned)(nch - 1);
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    if (par == 0) {
      float M = -INFINITY;
      for (int ch = 0; ch < nch; ++ch) {
        const int64_t it = ((int64_t)ch * p.ntiles * p.B + (int64_t)tile * p.B + b) * p.Hkv + kvh;
        M = fmaxf(M, p.partial[(it * kTileRows + rg * 32 + r32) * (D + 2) + D]);
      }
      const float Mu = M == -INFINITY ? 0.f : M;
      float Lsum = 0.f;
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[j][r] = 0.f;
      for (int ch = 0; ch < nch; ++ch) {
        const int64_t it = ((int64_t)ch * p.ntiles * p.B + (int64_t)tile * p.B + b) * p.Hkv + kvh;
        const float* pr = p.partial + (it * kTileRows + rg * 32 + r32) * (D + 2);
        const float w = __builtin_amdgcn_exp2f((pr[D] - Mu) * c);
        Lsum += pr[D + 1] * w;
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[j][r] += pr[NJ * (8 * (r / 4) + 4 * h + (r & 3)) + j] * w;
      }
      m = M;
      l = Lsum;
    }
    if (threadIdx.x == 0) p.counter[tile_id] = 0u;  // leave the counter clean
  }

  // ---- final normalisation and store
  if (par == 0 && row_ok) {
    const float inv = (kept && l > 0.f) ? 1.f / l : 0.f;
    uint16_t* orow = p.out + qrow * D;
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      // 4*NJ consecutive head dims start at NJ*(8*qd + 4h)
      uint32_t w[2 * NJ];
#pragma unroll
      for (int e = 0; e < 4 * NJ; e += 2) {
        const int r0 = 4 * qd + e / NJ, j0 = e % NJ;
        const int r1 = 4 * qd + (e + 1) / NJ, j1 = (e + 1) % NJ;
        w[e / 2] = f32_to_bf16(o[j0][r0] * inv) | (f32_to_bf16(o[j1][r1] * inv) << 16);
      }
      uint16_t* dst = orow + NJ * (8 * qd + 4 * h);
      *(u32x4*)dst = u32x4{w[0], w[1], w[2], w[3]};
      if constexpr (NJ == 4) *(u32x4*)(dst + 8) = u32x4{w[4], w[5], w[6], w[7]};
    }
    if (p.lse && h == 0) {
      const int64_t li = ((int64_t)b * p.Hq + qh) * ((int64_t)p.A * p.gamma) + (int64_t)ua * p.gamma + uk;
      p.lse[li] = (kept && l > 0.f) ? m * p.scale + kLn2 * __builtin_amdgcn_logf(l) : -INFINITY;
    }
  }
}

// ------------------------------------------------------ vector-ALU kernel
// float32 inputs (and any input the MFMA path does not take): one wave per
// (b, a, query head), rows of the block one after another, keys across lanes.
template <bool kBf16>
__global__ __launch_bounds__(64) void block_attn_valu(Params p, int D) {
  __shared__ float qs[128];
  __shared__ float ps[64];
  auto ld = [&](const void* base, int64_t i) -> float {
    return kBf16 ? __uint_as_float((uint32_t)((const uint16_t*)base)[i] << 16) : ((const float*)base)[i];
  };
  const int lane = threadIdx.x;
  int wid = blockIdx.x;
  const int h = wid % p.Hq; wid /= p.Hq;
  const int a = wid % p.A;
  const int b = wid / p.A;
  const int kvh = h / p.group;
  int c0, S;
  ctx_range(p, b, c0, S, a == 0 && h == 0 && lane == 0);
  int lim = visible_ctx(p, b, a, S, h == 0 && lane == 0);
  const bool kept = lim >= 0;
  if (!kept) lim = 0;
  const float c = p.scale * kLog2e;
  for (int k = 0; k < p.gamma; ++k) {
    const int64_t qrow = ((int64_t)b * p.A * p.gamma + (int64_t)a * p.gamma + k) * p.Hq + h;
    __syncthreads();
    for (int d = lane; d < D; d += 64) qs[d] = ld(p.q, qrow * D + d);
    __syncthreads();
    float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
    const int nkeys = kept ? lim + p.gamma : 0;
    for (int j0 = 0; j0 < nkeys; j0 += 64) {
      const int j = j0 + lane;
      float s = -INFINITY;
      int64_t row = 0;
      const void *kbp = nullptr, *vbp = nullptr;
      if (j < nkeys) {
        if (j < lim) { row = (int64_t)c0 + j; kbp = p.kc; vbp = p.vc; }
        else { row = (int64_t)b * p.A * p.gamma + (int64_t)a * p.gamma + (j - lim); kbp = p.kb; vbp = p.vb; }
        float acc = 0.f;
        for (int d = 0; d < D; ++d) acc = fmaf(qs[d], ld(kbp, (row * p.Hkv + kvh) * D + d), acc);
        s = acc;
      }
      float smax = s;
      for (int off = 32; off > 0; off >>= 1) smax = fmaxf(smax, __shfl_xor(smax, off, 64));
      const float mn = fmaxf(m, smax);
      const float mu = mn == -INFINITY ? 0.f : mn;
      const float alpha = __builtin_amdgcn_exp2f((m - mu) * c);
      const float pj = j < nkeys ? __builtin_amdgcn_exp2f((s - mu) * c) : 0.f;
      float psum = pj;
      for (int off = 32; off > 0; off >>= 1) psum += __shfl_xor(psum, off, 64);
      l = l * alpha + psum;
      m = mn;
      o0 *= alpha; o1 *= alpha;
      __syncthreads();
      ps[lane] = pj;
      __syncthreads();
      const int nj = min(64, nkeys - j0);
      for (int jj = 0; jj < nj; ++jj) {
        const int jg = j0 + jj;
        int64_t vr;
        const void* vp;
        if (jg < lim) { vr = (int64_t)c0 + jg; vp = p.vc; }
        else { vr = (int64_t)b * p.A * p.gamma + (int64_t)a * p.gamma + (jg - lim); vp = p.vb; }
        const float w = ps[jj];
        if (lane < D) o0 = fmaf(w, ld(vp, (vr * p.Hkv + kvh) * D + lane), o0);
        if (lane + 64 < D) o1 = fmaf(w, ld(vp, (vr * p.Hkv + kvh) * D + lane + 64), o1);
      }
    }
    const float inv = (kept && l > 0.f) ? 1.f / l : 0.f;
    if (kBf16) {
      uint16_t* o = (uint16_t*)p.out + qrow * D;
      if (lane < D) o[lane] = (uint16_t)f32_to_bf16(o0 * inv);
      if (lane + 64 < D) o[lane + 64] = (uint16_t)f32_to_bf16(o1 * inv);
    } else {
      float* o = (float*)p.out + qrow * D;
      if (lane < D) o[lane] = o0 * inv;
      if (lane + 64 < D) o[lane + 64] = o1 * inv;
    }
    if (p.lse && lane == 0) {
      const int64_t li = ((int64_t)b * p.Hq + h) * ((int64_t)p.A * p.gamma) + (int64_t)a * p.gamma + k;
      p.lse[li] = (kept && l > 0.f) ? m * p.scale + kLn2 * __builtin_amdgcn_logf(l) : -INFINITY;
    }
  }
}

__global__ void zero_u32_kernel(unsigned* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

struct Shape {
  int group, ntiles, nrows, nch_max;
  int64_t items;
};

Shape make_shape(int B, int A, int gamma, int Hq, int Hkv, int max_ctx) {
  Shape s{};
  s.group = Hq / Hkv;
  s.nrows = A * s.group * gamma;
  s.ntiles = (s.nrows + kTileRows - 1) / kTileRows;
  s.nch_max = max_ctx > 0 ? (max_ctx + kChunk - 1) / kChunk : 1;
  s.items = (int64_t)s.nch_max * s.ntiles * B * Hkv;
  return s;
}

}  // namespace

extern "C" size_t dspark_block_attention_workspace_bytes(int B, int A, int gamma, int Hq, int Hkv,
                                                         int D, int max_ctx) {
  if (B <= 0 || A <= 0 || gamma <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || D <= 0 || max_ctx < 0)
    return 0;
  const Shape s = make_shape(B, A, gamma, Hq, Hkv, max_ctx);
  const size_t part = s.nch_max > 1 ? (size_t)s.items * kTileRows * (D + 2) * sizeof(float) : 0;
  const size_t cnt = (size_t)s.ntiles * B * Hkv * sizeof(unsigned);
  return dspark_host::align_up(part, 256) + dspark_host::align_up(cnt, 256);
}

extern "C" int dspark_block_attention(const void* q, const void* k_ctx, const void* v_ctx,
                                      const int32_t* ctx_offsets, const void* k_blk,
                                      const void* v_blk, const int32_t* anchor_pos,
                                      const uint8_t* keep_mask, void* out, float* lse, int B,
                                      int A, int gamma, int Hq, int Hkv, int D, int max_ctx,
                                      int total_ctx, float scale, int dtype, void* ws,
                                      size_t ws_bytes, int32_t* dev_status, void* stream) {
  using namespace dspark_host;
  if (B < 0 || A < 0 || gamma < 0 || max_ctx < 0 || total_ctx < 0)
    return fail(DSPARK_ERR_INVALID_ARG, "block_attention: negative dimension");
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv)
    return fail(DSPARK_ERR_INVALID_ARG, "block_attention: need Hq %% Hkv == 0 (Hq=%d Hkv=%d)", Hq, Hkv);
  if (D != 64 && D != 128) return fail(DSPARK_ERR_INVALID_ARG, "block_attention: D must be 64 or 128 (got %d)", D);
  if (gamma > 64) return fail(DSPARK_ERR_INVALID_ARG, "block_attention: gamma > 64");
  if (dtype != DSPARK_BF16 && dtype != DSPARK_F32)
    return fail(DSPARK_ERR_INVALID_ARG, "block_attention: unknown dtype %d", dtype);
  if (!(scale > 0.f) || scale == INFINITY)
    return fail(DSPARK_ERR_INVALID_ARG, "block_attention: scale must be finite and > 0");
  if ((int64_t)B * A * gamma == 0) return ok();
  if ((int64_t)A * gamma * (Hq / Hkv) >= (1ll << 31) || (int64_t)B * A >= (1ll << 31))
    return fail(DSPARK_ERR_INVALID_ARG, "block_attention: row space too large");
  if (!q || !ctx_offsets || !k_blk || !v_blk || !anchor_pos || !keep_mask || !out ||
      (total_ctx > 0 && (!k_ctx || !v_ctx)))
    return fail(DSPARK_ERR_INVALID_ARG, "block_attention: null required pointer");
  hipStream_t s = (hipStream_t)stream;
  const Shape sh = make_shape(B, A, gamma, Hq, Hkv, max_ctx);
  Params p{};
  p.q = (const uint16_t*)q; p.kc = (const uint16_t*)k_ctx; p.vc = (const uint16_t*)v_ctx;
  p.offs = ctx_offsets; p.kb = (const uint16_t*)k_blk; p.vb = (const uint16_t*)v_blk;
  p.anchor = anchor_pos; p.keep = keep_mask; p.out = (uint16_t*)out; p.lse = lse;
  p.status = dev_status;
  p.B = B; p.A = A; p.gamma = gamma; p.Hq = Hq; p.Hkv = Hkv; p.group = sh.group;
  p.ntiles = sh.ntiles; p.nrows = sh.nrows; p.total_ctx = total_ctx; p.max_ctx = max_ctx;
  p.scale = scale;
  const bool aligned = ((uintptr_t)q | (uintptr_t)k_ctx | (uintptr_t)v_ctx | (uintptr_t)k_blk |
                        (uintptr_t)v_blk | (uintptr_t)out) % 16 == 0;
  if (dtype == DSPARK_BF16 && aligned) {
    const size_t need = dspark_block_attention_workspace_bytes(B, A, gamma, Hq, Hkv, D, max_ctx);
    if (ws_bytes < need || (need && !ws))
      return fail(DSPARK_ERR_WORKSPACE, "block_attention: workspace %zu bytes < %zu", ws_bytes, need);
    const size_t part = sh.nch_max > 1 ? (size_t)sh.items * kTileRows * (D + 2) * sizeof(float) : 0;
    p.partial = (float*)ws;
    p.counter = (unsigned*)((char*)ws + align_up(part, 256));
    const int64_t ncnt = (int64_t)sh.ntiles * B * Hkv;
    hipLaunchKernelGGL(zero_u32_kernel, dim3((unsigned)((ncnt + 255) / 256)), dim3(256), 0, s, p.counter, ncnt);
    if (sh.items >= (1ll << 31)) return fail(DSPARK_ERR_INVALID_ARG, "block_attention: grid too large");
    if (D == 128)
      hipLaunchKernelGGL(block_attn_mfma<128>, dim3((unsigned)sh.items), dim3(kThreads), 0, s, p);
    else
      hipLaunchKernelGGL(block_attn_mfma<64>, dim3((unsigned)sh.items), dim3(kThreads), 0, s, p);
  } else {
    const int64_t nb = (int64_t)B * A * Hq;
    if (nb >= (1ll << 31)) return fail(DSPARK_ERR_INVALID_ARG, "block_attention: grid too large");
    if (dtype == DSPARK_BF16)
      hipLaunchKernelGGL(block_attn_valu<true>, dim3((unsigned)nb), dim3(64), 0, s, p, D);
    else
      hipLaunchKernelGGL(block_attn_valu<false>, dim3((unsigned)nb), dim3(64), 0, s, p, D);
  }
  return check_launch("block_attention");
}
