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
// * One workgroup owns one tile for its whole key range: no split across
//   workgroups, so no partial results, counters or cache-maintenance fences.
//   A tile's context length is the largest anchor of its kept blocks; the
//   own-block keys of its blocks form extra 32-key slabs with a
//   block-diagonal mask, and per-score masking handles each block's anchor.
// * Load balance comes from the launch order: a one-workgroup planner sorts
//   the (request, tile) pairs by work, longest first (counting sort), and
//   the main grid walks that order, so the hardware's in-order dispatch is a
//   longest-processing-time schedule.  Within one rank the KV heads are
//   adjacent, so with 8 KV heads workgroup i runs on XCD i % 8 = kvh and
//   each XCD keeps one head's context K/V in its L2.
// * Four waves per workgroup: two 32-row groups x two key parities.  Per
//   32-key slab a wave computes S^T = K Q^T (v_mfma_f32_32x32x16_bf16; K rows
//   and Q rows are loaded as 16-byte row pieces), so each lane owns ONE query
//   row: the online-softmax max, sum and rescale are lane-local plus a single
//   cross-half exchange.  The probabilities feed O^T = V^T P^T straight from
//   the S^T accumulator layout (no transpose of P); V's head dimension is
//   permuted (slot m of product j is d = NJ*m + j) so every lane loads
//   NJ*2-byte pieces of key rows and transposes them in registers.
// * The slab loop is software-pipelined: the wave's next slab is loaded
//   (unconditionally, from clamped addresses, so the loads stay in flight
//   across the MFMA work) while the current one is computed.  Parities merge
//   through LDS at the end.
#include "common.h"

using namespace dspark;

namespace {

constexpr int kThreads = 256;
constexpr int kTileRows = 64;
constexpr int kPlanBins = 4096;  // cost buckets of the planner's counting sort
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
  const int32_t* order;  // launch order of tile ids (planner output)
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

// One 32-key slab as this lane holds it: K as the A operand of S^T (key slot
// r32, head dims 16*kk + 8h .. +7) and the V pieces of the 16 keys of its
// half (key of (t, s8) = 8*(2t + s8/4) + 4h + s8%4, head dims NJ*r32 .. +NJ-1).
template <int D>
struct Slab {
  u32x4 kf[D / 16];
  uint32_t v[2][8][D / 64];
};

// Per-workgroup constants of a work item.
struct Item {
  int64_t c0;        // first context row of the request
  int S;             // context length
  int cbeg, cend;    // context keys of this chunk
  int n_ctx_slabs;
  int64_t own0;      // first own-block row (k_blk / v_blk) of the tile's blocks
  int n_own;         // own-block keys of the tile
  int kvh, h, r32;
};

template <int D>
__device__ __forceinline__ void fetch_slab(const Params& p, const Item& it, int s, Slab<D>& sl) {
  constexpr int KK = D / 16, NJ = D / 32;
  const bool own = s >= it.n_ctx_slabs;
  const uint16_t* kbase = own ? p.kb : p.kc;
  const uint16_t* vbase = own ? p.vb : p.vc;
  int64_t krow;
  int j0 = 0, os = 0;
  if (!own) {
    j0 = it.cbeg + s * 32;
    krow = it.c0 + min(j0 + it.r32, it.S - 1);
  } else {
    os = (s - it.n_ctx_slabs) * 32;
    krow = it.own0 + min(os + it.r32, it.n_own - 1);
  }
  const uint16_t* kp = kbase + (krow * p.Hkv + it.kvh) * D + it.h * 8;
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) sl.kf[kk] = *(const u32x4*)(kp + kk * 16);
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) {
      const int ks = 8 * (2 * t + s8 / 4) + 4 * it.h + (s8 & 3);
      const int64_t vrow = own ? it.own0 + min(os + ks, it.n_own - 1) : it.c0 + min(j0 + ks, it.S - 1);
      const uint16_t* vp = vbase + (vrow * p.Hkv + it.kvh) * D + NJ * it.r32;
      if constexpr (NJ == 4) {
        const u32x2 w = *(const u32x2*)vp;
        sl.v[t][s8][0] = w.x;
        sl.v[t][s8][1] = w.y;
      } else {
        sl.v[t][s8][0] = *(const uint32_t*)vp;
      }
    }
}

// The running maximum of a row is only moved when a slab's maximum exceeds
// it by more than this many powers of two: the exponentials then stay below
// 2^kLazyMax (exact in float32, and in bf16 as precise as any probability),
// and most slabs skip the rescale of the accumulators entirely.
constexpr float kLazyMax = 8.f;

// Online-softmax update of this lane's row with one slab.
template <int D>
__device__ __forceinline__ void compute_slab(const Params& p, const Item& it, int s, const Slab<D>& sl,
                                             const u32x4* qf, bool kept, int lim, int ua, int a_lo,
                                             float c, float& m, float& l, f32x16* o) {
  constexpr int KK = D / 16, NJ = D / 32;
  const bool own = s >= it.n_ctx_slabs;
  const int j0 = own ? 0 : it.cbeg + s * 32;
  const int os = own ? (s - it.n_ctx_slabs) * 32 : 0;
  f32x16 sc;
#pragma unroll
  for (int i = 0; i < 16; ++i) sc[i] = 0.f;
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) sc = mfma32x32x16(sl.kf[kk], qf[kk], sc);
  // context slabs that every row of the wave sees whole need no masking
  const bool whole = !own && kept && j0 + 32 <= min(it.cend, lim);
  if (!__all(whole)) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int ks = 8 * (i / 4) + 4 * it.h + (i & 3);
      bool vis;
      if (!own) {
        const int j = j0 + ks;
        vis = kept && j < it.cend && j < lim;
      } else {
        const int o_i = os + ks;
        vis = kept && o_i < it.n_own && (a_lo + o_i / p.gamma) == ua;
      }
      sc[i] = vis ? sc[i] : -INFINITY;
    }
  }
  float smax = sc[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) smax = fmaxf(smax, sc[i]);
  smax = fmaxf(smax, __shfl_xor(smax, 32, kWave));
  // lazy maximum: move it (and rescale) only when this slab would push the
  // exponentials past 2^kLazyMax
  const bool grow = smax > m && (m == -INFINITY || (smax - m) * c > kLazyMax);
  if (__any(grow)) {
    const float mnew = grow ? smax : m;
    const float alpha = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m - mnew) * c);
    l *= alpha;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[j][r] *= alpha;
    m = mnew;
  }
  const float mc = m == -INFINITY ? 0.f : m * c;
  float psum = 0.f;
  u32x4 pb[2];
#pragma unroll
  for (int i = 0; i < 16; i += 2) {
    const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[i], c, -mc));
    const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[i + 1], c, -mc));
    psum += p0 + p1;
    pb[i / 8][(i % 8) / 2] = pack_bf16x2(p0, p1);
  }
  psum += __shfl_xor(psum, 32, kWave);
  l += psum;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      u32x4 va;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t lo = sl.v[t][2 * w][j / 2], hi = sl.v[t][2 * w + 1][j / 2];
        va[w] = (j & 1) ? pack_hi(lo, hi) : pack_lo(lo, hi);
      }
      o[j] = mfma32x32x16(va, pb[t], o[j]);
    }
  }
}

// Head dim of accumulator register r of product j for a lane in half h.
template <int NJ>
__device__ __forceinline__ int head_dim(int r, int j, int h) { return NJ * (8 * (r / 4) + 4 * h + (r & 3)) + j; }

// Work of a (request, tile) pair in 32-key slabs (context + own keys); -1
// when none of its blocks is kept.
__device__ __forceinline__ int tile_cost(const Params& p, int b, int tile, int& L, int& a_lo, int& a_hi,
                                         bool& any_kept) {
  int c0, S;
  ctx_range(p, b, c0, S, false);
  const int rpb = p.group * p.gamma;
  const int u0 = tile * kTileRows;
  a_lo = u0 / rpb;
  a_hi = min(p.A - 1, (u0 + kTileRows - 1) / rpb);
  L = 0;
  any_kept = false;
  for (int a = a_lo; a <= a_hi; ++a) {
    const int v = visible_ctx(p, b, a, S, false);
    if (v >= 0) { any_kept = true; L = max(L, v); }
  }
  const int n_own = (a_hi - a_lo + 1) * p.gamma;
  return any_kept ? (L + 31) / 32 + (n_own + 31) / 32 : 0;
}

// Longest-first launch order: counting sort of the B*ntiles (request, tile)
// pairs by cost, descending; entry r*Hkv + kvh of `order` is the tile id
// (pair * Hkv + kvh).  Ties are ordered arbitrarily (results do not depend
// on the order, only the schedule does).
__global__ __launch_bounds__(1024) void attn_plan_kernel(Params p, int32_t* __restrict__ order) {
  __shared__ int hist[kPlanBins];
  __shared__ int part[1024];
  const int npairs = p.B * p.ntiles;
  for (int i = threadIdx.x; i < kPlanBins; i += 1024) hist[i] = 0;
  __syncthreads();
  for (int q = threadIdx.x; q < npairs; q += 1024) {
    int L, a_lo, a_hi;
    bool any;
    const int cost = tile_cost(p, q % p.B, q / p.B, L, a_lo, a_hi, any);
    atomicAdd(&hist[min(cost, kPlanBins - 1)], 1);
  }
  __syncthreads();
  // exclusive scan in descending bin order: thread t owns bins 4095-4t .. 4092-4t
  int local = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) local += hist[kPlanBins - 1 - 4 * threadIdx.x - k];
  part[threadIdx.x] = local;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int t = 0; t < 1024; ++t) { const int v = part[t]; part[t] = run; run += v; }
  }
  __syncthreads();
  int run = part[threadIdx.x];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int bin = kPlanBins - 1 - 4 * threadIdx.x - k;
    const int v = hist[bin];
    hist[bin] = run;
    run += v;
  }
  __syncthreads();
  for (int q = threadIdx.x; q < npairs; q += 1024) {
    int L, a_lo, a_hi;
    bool any;
    const int cost = tile_cost(p, q % p.B, q / p.B, L, a_lo, a_hi, any);
    const int pos = atomicAdd(&hist[min(cost, kPlanBins - 1)], 1);
    const int b = q % p.B, tile = q / p.B;
    for (int kvh = 0; kvh < p.Hkv; ++kvh)
      order[(int64_t)pos * p.Hkv + kvh] = ((tile * p.B) + b) * p.Hkv + kvh;
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) void block_attn_mfma(Params p) {
  constexpr int NJ = D / 32;  // head-dim groups of the PV product
  constexpr int KK = D / 16;  // k-steps of the QK product
  __shared__ float mrg[2][D + 2][32];

  // ---- decode the work item (tile id = (tile * B + b) * Hkv + kvh)
  int wid = p.order ? p.order[blockIdx.x] : (int)blockIdx.x;
  const int kvh = wid % p.Hkv; wid /= p.Hkv;
  const int b = wid % p.B;
  const int tile = wid / p.B;
  int c0, S;
  ctx_range(p, b, c0, S, tile == 0 && kvh == 0 && threadIdx.x == 0);
  int L, a_lo, a_hi;
  bool any_kept;
  tile_cost(p, b, tile, L, a_lo, a_hi, any_kept);
  const int rpb = p.group * p.gamma;
  const int u0 = tile * kTileRows;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int rg = wave & 1, par = wave >> 1;
  const int h = lane >> 5, r32 = lane & 31;
  // this lane's query row (rows past the row space are computed on a clamped
  // row and not stored)
  const int u = u0 + rg * 32 + r32;
  const bool row_ok = u < p.nrows;
  const int uc = min(u, p.nrows - 1);
  const int ua = uc / rpb;
  const int uhg = (uc / p.gamma) % p.group, uk = uc % p.gamma;
  const int qh = kvh * p.group + uhg;
  int lim = visible_ctx(p, b, ua, S, par == 0 && h == 0 && row_ok);
  const bool kept = row_ok && lim >= 0;
  if (!kept) lim = 0;
  const int64_t qrow = ((int64_t)b * p.A * p.gamma + (int64_t)ua * p.gamma + uk) * p.Hq + qh;

  // Q^T operand pieces: d = 16*kk + 8*h .. +7
  u32x4 qf[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) qf[kk] = *(const u32x4*)(p.q + qrow * D + kk * 16 + h * 8);

  Item it;
  it.c0 = c0; it.S = S;
  it.cbeg = 0;
  it.cend = L;
  it.n_ctx_slabs = (L + 31) / 32;
  it.own0 = (int64_t)b * p.A * p.gamma + (int64_t)a_lo * p.gamma;
  it.n_own = (a_hi - a_lo + 1) * p.gamma;
  it.kvh = kvh; it.h = h; it.r32 = r32;
  const int nslab = any_kept ? it.n_ctx_slabs + (it.n_own + 31) / 32 : 0;
  const float c = p.scale * kLog2e;

  float m = -INFINITY, l = 0.f;
  f32x16 o[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[j][r] = 0.f;

  // ---- slab loop, software-pipelined: the wave's next slab is in flight
  //      while the current one is computed (the prefetch index is clamped so
  //      the loads are unconditional)
  if (par < nslab) {
    Slab<D> sa, sb;
    fetch_slab<D>(p, it, par, sa);
    for (int s = par; s < nslab; s += 4) {
      fetch_slab<D>(p, it, min(s + 2, nslab - 1), sb);
      compute_slab<D>(p, it, s, sa, qf, kept, lim, ua, a_lo, c, m, l, o);
      if (s + 2 >= nslab) break;
      fetch_slab<D>(p, it, min(s + 4, nslab - 1), sa);
      compute_slab<D>(p, it, s + 2, sb, qf, kept, lim, ua, a_lo, c, m, l, o);
    }
  }

  // ---- merge the two key parities of each row group through LDS
  if (par == 1) {
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) mrg[rg][head_dim<NJ>(r, j, h)][r32] = o[j][r];
    if (h == 0) { mrg[rg][D][r32] = m; mrg[rg][D + 1][r32] = l; }
  }
  __syncthreads();
  if (par == 1 || !row_ok) return;
  {
    const float m1 = mrg[rg][D][r32], l1 = mrg[rg][D + 1][r32];
    const float mn = fmaxf(m, m1);
    const float mu = mn == -INFINITY ? 0.f : mn;
    const float a0 = __builtin_amdgcn_exp2f((m - mu) * c), a1 = __builtin_amdgcn_exp2f((m1 - mu) * c);
    l = l * a0 + l1 * a1;
    m = mn;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[j][r] = o[j][r] * a0 + mrg[rg][head_dim<NJ>(r, j, h)][r32] * a1;
  }

  // ---- final normalisation and store
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
      w[e / 2] = pack_bf16x2(o[j0][r0] * inv, o[j1][r1] * inv);
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

struct Shape {
  int group, ntiles, nrows;
  int64_t tiles;  // B * ntiles * Hkv
};

Shape make_shape(int B, int A, int gamma, int Hq, int Hkv) {
  Shape s{};
  s.group = Hq / Hkv;
  s.nrows = A * s.group * gamma;
  s.ntiles = (s.nrows + kTileRows - 1) / kTileRows;
  s.tiles = (int64_t)s.ntiles * B * Hkv;
  return s;
}

}  // namespace

extern "C" size_t dspark_block_attention_workspace_bytes(int B, int A, int gamma, int Hq, int Hkv,
                                                         int D, int max_ctx) {
  (void)D; (void)max_ctx;
  if (B <= 0 || A <= 0 || gamma <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || max_ctx < 0) return 0;
  const Shape s = make_shape(B, A, gamma, Hq, Hkv);
  return dspark_host::align_up((size_t)s.tiles * sizeof(int32_t), 256);
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
  const Shape sh = make_shape(B, A, gamma, Hq, Hkv);
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
    if (sh.tiles >= (1ll << 31)) return fail(DSPARK_ERR_INVALID_ARG, "block_attention: grid too large");
    int32_t* order = (int32_t*)ws;
    hipLaunchKernelGGL(attn_plan_kernel, dim3(1), dim3(1024), 0, s, p, order);
    p.order = order;
    if (D == 128)
      hipLaunchKernelGGL(block_attn_mfma<128>, dim3((unsigned)sh.tiles), dim3(kThreads), 0, s, p);
    else
      hipLaunchKernelGGL(block_attn_mfma<64>, dim3((unsigned)sh.tiles), dim3(kThreads), 0, s, p);
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
