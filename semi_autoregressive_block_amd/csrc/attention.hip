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
//   u = (a * group + hg) * gamma + k and cut into tiles of 64 or 128 rows,
//   so one tile packs several heads (and, for short blocks, several
//   consecutive blocks) against the same keys: the MFMA M/N extent is
//   filled by GQA packing, not by padding gamma.
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
// * Two tile heights.  When a context is read by at most two 64-row tiles
//   per KV head (serving: one block per request) it streams from HBM once:
//   64-row tiles.  When many tiles re-read it (all-anchor training) it comes
//   from L2: 128-row tiles, so each staged slab serves twice the rows.
//   Either way two workgroups of four waves share a compute unit.
// * Per 32-key slab a wave computes S^T = K Q^T (v_mfma_f32_32x32x16_bf16),
//   so each lane owns ONE query row: the online-softmax max, sum and rescale
//   are lane-local plus a single cross-half exchange (v_permlane32_swap).
//   The probabilities feed O^T = V^T P^T straight from the S^T accumulator
//   layout (no transpose of P); V^T operands come from transposing LDS reads.
// * Keys go in pairs of 32-key slabs.  64-row tiles: waves are 32-row groups
//   x two key parities (one slab of each pair per wave; the parities merge
//   through LDS at the end), so a streaming tile still has four waves.
//   128-row tiles: one wave per 32-row group takes both slabs of a pair: two
//   S^T chains back to back, then a softmax step and P.V product per slab,
//   so the vector and matrix work of the two slabs overlap within the wave.
// * K/V staging: each pair goes straight from global memory into a two-slot
//   ring in LDS (direct LDS loads: no register round trip).
#include "common.h"

using namespace dspark;

namespace {

constexpr int kTileRows = 64;  // rows per tile of the streaming kernel and of the workspace
constexpr int kPlanBins = 4096;  // cost buckets of the planner's counting sort
constexpr int kPlanCache = 16384;  // (request, tile) pairs whose bins the planner keeps in LDS
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
  int tile_rows;                                    // rows per tile (64 or 128)
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
  // both loads go out together (one round trip, not two)
  const uint8_t kp = p.keep[(int64_t)b * p.A + a];
  const int an = p.anchor[(int64_t)b * p.A + a];
  if (!kp) return -1;  // masked block
  if (flag && (an < 0 || an > S)) status_or(p.status, DSPARK_STATUS_BAD_ANCHOR);
  return clampi(an, 0, S);
}


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

// x combined with the value of lane x ^ 32, in every lane: v_permlane32_swap
// of x with itself leaves the low half's value in one result and the high
// half's in the other.
__device__ __forceinline__ float half_combine_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_combine_add(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The running maximum of a row is only moved when a slab's maximum exceeds
// it by more than this many powers of two: the exponentials then stay below
// 2^kLazyMax (exact in float32, and in bf16 as precise as any probability),
// and most slabs skip the rescale of the accumulators entirely.
constexpr float kLazyMax = 8.f;

// S^T of one slab: key slot i of accumulator register i's row, this lane's
// query row as the column.
template <int D, class Src>
__device__ __forceinline__ f32x16 qk_slab(const Src& sl, const u32x4* qf) {
  f32x16 sc;
#pragma unroll
  for (int i = 0; i < 16; ++i) sc[i] = 0.f;
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) sc = mfma32x32x16(sl.k(kk), qf[kk], sc);
  return sc;
}

// Scores of slab s that this lane's row may not see become -inf: context
// keys below min(chunk end, anchor), own keys of its block only (one gamma
// range).  Slabs that every row of the wave sees whole are left alone.
__device__ __forceinline__ void mask_scores(const Params& p, const Item& it, int s, bool kept, int lim, int ua,
                                            int a_lo, f32x16& sc) {
  const bool own = s >= it.n_ctx_slabs;
  const int j0 = own ? 0 : it.cbeg + s * 32;
  const int os = own ? (s - it.n_ctx_slabs) * 32 : 0;
  int vlo, vhi;  // visible key slots: vlo <= slot < vhi
  if (!own) {
    vlo = -1 - j0;
    vhi = kept ? min(it.cend, lim) - j0 : 0;
  } else {
    vlo = (ua - a_lo) * p.gamma - os;
    vhi = kept ? vlo + p.gamma : vlo;
  }
  if (!__all(vlo <= 0 && vhi >= 32)) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int ks = 8 * (i / 4) + 4 * it.h + (i & 3);
      sc[i] = (ks >= vlo && ks < vhi) ? sc[i] : -INFINITY;
    }
  }
}

// Online-softmax update of this lane's row with the scores sc of slab s.
template <int D, class Src>
__device__ __forceinline__ void softmax_pv(const Params& p, const Item& it, int s, f32x16 sc, const Src& sl,
                                           bool kept, int lim, int ua, int a_lo, float c, float& m, float& l,
                                           f32x16* o) {
  constexpr int NJ = D / 32;
  mask_scores(p, it, s, kept, lim, ua, a_lo, sc);
  float smax = sc[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) smax = fmaxf(smax, sc[i]);
  smax = half_combine_max(smax);
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
  psum = half_combine_add(psum);
  l += psum;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) o[j] = mfma32x32x16(sl.v(t, j), pb[t], o[j]);
  }
}

template <int D, class Src>
__device__ __forceinline__ void compute_slab(const Params& p, const Item& it, int s, const Src& sl,
                                             const u32x4* qf, bool kept, int lim, int ua, int a_lo,
                                             float c, float& m, float& l, f32x16* o) {
  softmax_pv<D>(p, it, s, qk_slab<D>(sl, qf), sl, kept, lim, ua, a_lo, c, m, l, o);
}

// Both slabs of a pair (s0 and s0 + 1) for one wave.  The two S^T products
// go out back to back as two chains (slab s0's first), then each slab takes
// its own online-softmax step and P.V product: slab s0's exponentials run
// while the matrix cores still work on slab s0 + 1's S^T, and slab s0 + 1's
// exponentials while they work on slab s0's P.V.  A pair past the last slab
// (odd slab count) has no second step; its ring copy repeats the last slab.
// after_qk() runs once the S^T products are issued (the caller's ring refill:
// a copy that stalls on a full load queue then overlaps matrix work).
template <int D, class Src, class AfterQK>
__device__ __forceinline__ void compute_pair(const Params& p, const Item& it, int s0, int nslab, const Src& sa,
                                             const Src& sb, const u32x4* qf, bool kept, int lim, int ua,
                                             int a_lo, float c, float& m, float& l, f32x16* o,
                                             AfterQK after_qk) {
  constexpr int NJ = D / 32;
  constexpr int KK = D / 16;
  f32x16 x, y;
#pragma unroll
  for (int i = 0; i < 16; ++i) { x[i] = 0.f; y[i] = 0.f; }
  // Slab s0's K operands are read one rank step ahead of its products (two
  // operand sets) and slab s0 + 1's all during them; the scheduling groups
  // below pin that order, which the scheduler would otherwise fold back to
  // read-wait-multiply.
  // The products go out at raised priority: when both waves of a SIMD are
  // ready, the one that feeds the matrix cores issues first.
  u32x4 kx[2], ky[KK];
  __builtin_amdgcn_s_setprio(1);
  kx[0] = sa.k(0);
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    if (kk + 1 < KK) kx[(kk + 1) & 1] = sa.k(kk + 1);
    x = mfma32x32x16(kx[kk & 1], qf[kk], x);
    ky[kk] = sb.k(kk);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // first read of slab s0
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    if (kk + 1 < KK) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // next read of s0
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                   // product kk of s0
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                   // read kk of s0 + 1
  }
  // slab s0's last product is used here, so it cannot sink below slab
  // s0 + 1's chain (it would delay slab s0's softmax step by a whole chain)
  asm volatile("" ::"v"(x[0]));
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) y = mfma32x32x16(ky[kk], qf[kk], y);
  __builtin_amdgcn_s_setprio(0);
  after_qk();
  float psum = 0.f;
  auto step = [&](f32x16& sc, int s, const Src& sl) {
    mask_scores(p, it, s, kept, lim, ua, a_lo, sc);
    float smax = sc[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) smax = fmaxf(smax, sc[i]);
    smax = half_combine_max(smax);
    const bool grow = smax > m && (m == -INFINITY || (smax - m) * c > kLazyMax);
    if (__any(grow)) {
      const float mnew = grow ? smax : m;
      const float alpha = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m - mnew) * c);
      l *= alpha;
      psum *= alpha;
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[j][r] *= alpha;
      m = mnew;
    }
    const float mc = m == -INFINITY ? 0.f : m * c;
    u32x4 pb[2];
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[i], c, -mc));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[i + 1], c, -mc));
      psum += p0 + p1;
      pb[i / 8][(i % 8) / 2] = pack_bf16x2(p0, p1);
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int j = 0; j < NJ; ++j) o[j] = mfma32x32x16(sl.v(t, j), pb[t], o[j]);
  };
  step(x, s0, sa);
  if (s0 + 1 < nslab) step(y, s0 + 1, sb);  // uniform
  l += half_combine_add(psum);
}

// Head dim of accumulator register r of product j for a lane in half h.
__device__ __forceinline__ int head_dim(int r, int j, int h) { return 32 * j + 8 * (r / 4) + 4 * h + (r & 3); }

// Work of a (request, tile) pair in 32-key slabs (context + own keys); -1
// when none of its blocks is kept.
__device__ __forceinline__ int tile_cost(const Params& p, int b, int tile, int& L, int& a_lo, int& a_hi,
                                         bool& any_kept) {
  int c0, S;
  ctx_range(p, b, c0, S, false);
  const int rpb = p.group * p.gamma;
  const int u0 = tile * p.tile_rows;
  a_lo = u0 / rpb;
  a_hi = min(p.A - 1, (u0 + p.tile_rows - 1) / rpb);
  L = 0;
  any_kept = false;
  // four blocks' keep flags and anchors per round trip
  const int64_t r0 = (int64_t)b * p.A;
  for (int a0 = a_lo; a0 <= a_hi; a0 += 4) {
    uint8_t kp[4];
    int an[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int a = min(a0 + j, a_hi);
      kp[j] = p.keep[r0 + a];
      an[j] = p.anchor[r0 + a];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (a0 + j <= a_hi && kp[j]) { any_kept = true; L = max(L, clampi(an[j], 0, S)); }
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
  __shared__ int wsum[16];
  __shared__ uint16_t cached[kPlanCache];  // bin of pair q (when npairs <= kPlanCache)
  const int npairs = p.B * p.ntiles;
  const bool cache = npairs <= kPlanCache;
  for (int i = threadIdx.x; i < kPlanBins; i += 1024) hist[i] = 0;
  __syncthreads();
  for (int q = threadIdx.x; q < npairs; q += 1024) {
    int L, a_lo, a_hi;
    bool any;
    const int bin = min(tile_cost(p, q % p.B, q / p.B, L, a_lo, a_hi, any), kPlanBins - 1);
    if (cache) cached[q] = (uint16_t)bin;
    atomicAdd(&hist[bin], 1);
  }
  __syncthreads();
  // exclusive scan in descending bin order: thread t owns bins 4095-4t ..
  // 4092-4t; wave prefix sums, then the 16 wave totals
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int local = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) local += hist[kPlanBins - 1 - 4 * threadIdx.x - k];
  int incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  int run = before + incl - local;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int bin = kPlanBins - 1 - 4 * threadIdx.x - k;
    const int v = hist[bin];
    hist[bin] = run;
    run += v;
  }
  __syncthreads();
  for (int q = threadIdx.x; q < npairs; q += 1024) {
    int bin;
    if (cache) {
      bin = cached[q];
    } else {
      int L, a_lo, a_hi;
      bool any;
      bin = min(tile_cost(p, q % p.B, q / p.B, L, a_lo, a_hi, any), kPlanBins - 1);
    }
    const int pos = atomicAdd(&hist[bin], 1);
    const int b = q % p.B, tile = q / p.B;
    for (int kvh = 0; kvh < p.Hkv; ++kvh)
      order[(int64_t)pos * p.Hkv + kvh] = ((tile * p.B) + b) * p.Hkv + kvh;
  }
}

// ------------------------------------------------------------ MFMA kernel
// K and V reach the waves through LDS: the workgroup's waves copy each pair
// of 32-key slabs (one per key parity) together, as 16-byte pieces, into a
// ring slot, so a slab is fetched once per workgroup and read by all its row
// groups.  K rows are stored with their 16-byte pieces XOR-swizzled by the
// key index, so the MFMA-operand reads (one piece of 32 different keys) hit
// distinct LDS banks; V rows have their 64-byte groups XOR-rotated by the
// key, for the transposing reads.
template <int D>
struct Ring {
  static constexpr int kPieces = D * 2 / 16;             // 16-byte pieces per key row
  static constexpr int kTensorBytes = 32 * D * 2;        // K (or V) of one slab
  static constexpr int kSlotBytes = 2 * kTensorBytes;    // parity-0 slab then parity-1 slab
  // The XOR term of key row `key`.  A 16-byte read is served sixteen lanes (256 bytes, every
  // bank once) at a time, and lanes 0-15 read keys 0-15: 256-byte rows (D = 128) XOR the piece
  // with key mod 16; 128-byte rows (D = 64) sit two to a bank line, so keys 2m and 2m + 1 take
  // the two halves and the piece is XORed with m mod 8.
  __device__ static constexpr int ksw(int key) { return kPieces >= 16 ? key % kPieces : (key >> 1) % kPieces; }
  // The rotation of key row `key`'s 64-byte V groups.  A transposing read's 32 lanes take 64 bytes
  // of each of four keys 4m .. 4m + 3: 256-byte rows rotate by key mod 4; 128-byte rows (two to a
  // bank line) rotate by (key >> 1) mod 2, so keys 4m + 1 and 4m + 3 sit in the other half.
  static constexpr int kGroups = kPieces / 4;            // 64-byte groups per key row
  __device__ static constexpr int vsw(int key) { return kGroups >= 4 ? key % kGroups : (key >> 1) % kGroups; }
};

// Where a workgroup's slabs come from (wave-uniform): slab s < n_ctx_slabs
// is context keys 32s .. 32s+31 from ctx_row0, later slabs are the tile's
// own block keys from own_row0.  Keys past a source's last row are read
// from that last row (they are masked in the scores).
struct SlabSource {
  const unsigned char *kc, *vc, *kb, *vb;
  int64_t ctx_row0, own_row0;  // first row of the context chunk / of the tile's own keys
  int ctx_keys, own_keys, n_ctx_slabs, nslab;
  uint32_t row_b;              // bytes between consecutive rows (all heads)
  uint32_t head_b;             // byte offset of this KV head inside a row
};

// This lane's operand pieces of one staged slab.  K piece kk (key r32, head
// dims 16*kk + 8h .. +7) sits at chunk r32*P + ((2kk + h) ^ ksw(r32)) =
// r32*P + (2kk ^ y), y = h ^ ksw(r32).  V^T comes from ds_read_b64_tr_b16:
// in each 16-lane group, lane l receives element l mod 4 of the 8 bytes
// addressed by lane 4e + l/4, as its element e.  So when lane l (= r32 mod
// 16) addresses key kb + l/4, head dims d0 + 4(l mod 4) .. +3, it receives
// keys kb .. kb+3 of head dim d0 + l: with d0 = 32j + 16(r32/16) and
// kb = 16t + 4h (+8 for the second read) that is its V^T operand.
template <int D>
struct SlabView {
  using Rg = Ring<D>;
  static constexpr int P = Rg::kPieces;
  const unsigned char *kp, *vp;  // this slab's K and V in the rings
  uint32_t kbase, kx;            // K: lane row, XOR term
  uint32_t vbase, vx;            // V: lane part of the address, XOR term of the 64-byte group
  __device__ SlabView(const unsigned char* kslab, const unsigned char* vslab, int h, int r32)
      : kp(kslab), vp(vslab) {
    kbase = r32 * P * 16;
    kx = (h ^ Rg::ksw(r32)) * 16;
    const int l = r32 % 16, g2 = r32 / 16;
    const int key = 4 * h + l / 4;  // plus 16t + 8e
    vbase = key * (D * 2) + 32 * g2 + 8 * (l % 4);
    vx = 64 * Rg::vsw(l / 4);  // the group rotation of key 4h + l/4 (+16t + 8e: same low two bits)
  }
  __device__ u32x4 k(int kk) const { return *(const u32x4*)(kp + kbase + ((32 * kk) ^ kx)); }
  __device__ u32x4 v(int t, int j) const {
    typedef short i16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const unsigned char* a = vp + vbase + ((64 * j) ^ vx) + 16 * t * (D * 2);
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)a);
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a + 8 * (D * 2)));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    return u32x4{l2.x, l2.y, h2.x, h2.y};
  }
};


// K/V staging straight from global memory into LDS (global_load_lds_dwordx4,
// no register round trip): one instruction moves 64 lanes x 16 bytes into
// 1 KB of LDS, lane l to chunk base + l, so each lane fetches the piece
// that the K or V swizzle puts at that chunk.  A ring slot holds one pair:
// K of both parities, then V of both parities.  The compiler does not
// order these LDS writes against LDS reads: the consumer waits for its own
// copies with an explicit vmcnt and then meets the other waves at a plain
// s_barrier (no fence, which would wait for every copy in flight).
template <int D, int NT>
struct DmaPair {
  using Rg = Ring<D>;
  static constexpr int P = Rg::kPieces;
  static constexpr int kInst = Rg::kSlotBytes / 1024;  // 1 KB copies per half (K or V) of a pair
  static constexpr int kPerWave = kInst / (NT / 64);
  static constexpr int kPerPair = 2 * kPerWave;         // copies per wave per pair
  static_assert(kInst % (NT / 64) == 0 && (32 * P) % 64 == 0, "copy layout");
  __device__ static void issue(const SlabSource& st, int pair, unsigned char* slot, int wave, int lane) {
#pragma unroll
    for (int hv = 0; hv < 2; ++hv)
#pragma unroll
      for (int j = 0; j < kPerWave; ++j) {
        const int inst = wave * kPerWave + j;     // wave-uniform
        const int q = (inst * 64) / (32 * P);     // slab parity of this copy
        const int cc = (inst * 64) % (32 * P) + lane;  // chunk within the slab
        const int key = cc / P;
        const int piece = (cc % P) ^ (hv ? 4 * Rg::vsw(key) : Rg::ksw(key));
        const int s = min(2 * pair + q, st.nslab - 1);
        const bool own = s >= st.n_ctx_slabs;
        const int k0 = own ? (s - st.n_ctx_slabs) * 32 : s * 32;
        const int nvalid = (own ? st.own_keys : st.ctx_keys) - k0;
        const unsigned char* src = hv ? (own ? st.vb : st.vc) : (own ? st.kb : st.kc);
        src += ((own ? st.own_row0 : st.ctx_row0) + k0) * (int64_t)st.row_b + st.head_b;
        const uint32_t off = __umul24((uint32_t)min(key, nvalid - 1), st.row_b) + piece * 16;
        __builtin_amdgcn_global_load_lds((const void*)(src + off),
                                         (__attribute__((address_space(3))) void*)(slot + hv * Rg::kSlotBytes + inst * 1024),
                                         16, 0, 0);
      }
  }
};

// One workgroup per tile of 32*RG query rows and one (request, KV head):
// RG row groups x two key parities, one wave each; direct-to-LDS copies into
// an NSLOT-slot ring keep the next NSLOT - 1 slab pairs in flight.
template <int D, int RG, int NSLOT, int NPAR>
__global__ __launch_bounds__(64 * NPAR * RG) __attribute__((amdgpu_waves_per_eu(2, 2))) void block_attn_mfma(Params p) {
  using Rg = Ring<D>;
  constexpr int NJ = D / 32;
  constexpr int KK = D / 16;
  constexpr int NT = 64 * NPAR * RG;  // RG row groups x NPAR key parities, one wave each
  constexpr int kMergeBytes = NPAR == 2 ? RG * (D + 2) * 32 * 4 : 0;
  static_assert(NSLOT >= 2, "at least one pair in flight");
  static_assert(NPAR == 1 || NPAR == 2, "one wave per pair or per slab");
  constexpr int kRingBytes = NSLOT * 2 * Rg::kSlotBytes;
  __shared__ __align__(16) unsigned char ring[kRingBytes > kMergeBytes ? kRingBytes : kMergeBytes];

  // the work item is the same for the whole workgroup: keep it in scalars
  int wid = __builtin_amdgcn_readfirstlane(p.order ? p.order[blockIdx.x] : (int)blockIdx.x);
  const int kvh = wid % p.Hkv; wid /= p.Hkv;
  const int b = wid % p.B;
  const int tile = wid / p.B;
  int c0, S;
  ctx_range(p, b, c0, S, tile == 0 && kvh == 0 && threadIdx.x == 0);
  c0 = __builtin_amdgcn_readfirstlane(c0);
  S = __builtin_amdgcn_readfirstlane(S);
  int L, a_lo, a_hi;
  bool any_kept;
  tile_cost(p, b, tile, L, a_lo, a_hi, any_kept);
  L = __builtin_amdgcn_readfirstlane(L);
  a_lo = __builtin_amdgcn_readfirstlane(a_lo);
  a_hi = __builtin_amdgcn_readfirstlane(a_hi);
  any_kept = __builtin_amdgcn_readfirstlane((int)any_kept) != 0;
  const int rpb = p.group * p.gamma;
  const int u0 = tile * p.tile_rows;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rg = wave % RG, par = NPAR == 2 ? wave / RG : 0;
  const int h = lane >> 5, r32 = lane & 31;
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
  const int npairs = (nslab + 1) / 2;
  const float c = p.scale * kLog2e;

  SlabSource st;
  {
    st.kc = (const unsigned char*)p.kc; st.vc = (const unsigned char*)p.vc;
    st.kb = (const unsigned char*)p.kb; st.vb = (const unsigned char*)p.vb;
    st.ctx_row0 = (int64_t)c0 + it.cbeg;
    st.own_row0 = it.own0;
    st.ctx_keys = S - it.cbeg;  // rows past the context end repeat its last row
    st.own_keys = it.n_own;
    st.n_ctx_slabs = it.n_ctx_slabs;
    st.nslab = nslab;
    st.row_b = (uint32_t)p.Hkv * D * 2;
    st.head_b = (uint32_t)kvh * D * 2;
  }

  float m = -INFINITY, l = 0.f;
  f32x16 o[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[j][r] = 0.f;

  {
    // ---- pair i is computed from slot i mod NSLOT while pairs i+1 ..
    //      i+NSLOT-1 are being copied in.  Iteration i: wait for this wave's
    //      copies of pair i, meet the other waves (their copies of pair i
    //      are in, and they are done with pair i-1, whose slot is refilled
    //      next), compute pair i and issue pair i+NSLOT-1 (before the
    //      products of a parity wave, after the S^T products of a pair
    //      wave).  Copies past the end
    //      repeat the last slab (from L2), so the count is exact.
    using Dp = DmaPair<D, NT>;
    auto dslot = [&](int i) { return ring + (i % NSLOT) * 2 * Rg::kSlotBytes; };
    auto dview = [&](int i, int q) {
      unsigned char* sl = dslot(i);
      return SlabView<D>(sl + q * Rg::kTensorBytes, sl + Rg::kSlotBytes + q * Rg::kTensorBytes, h, r32);
    };
    if (npairs > 0) {
#pragma unroll
      for (int q = 0; q < NSLOT - 1; ++q) Dp::issue(st, q, dslot(q), wave, lane);
      for (int i = 0; i < npairs; ++i) {
        wait_vmcnt<Dp::kPerPair * (NSLOT - 2)>();
        block_barrier();
        auto refill = [&]() { Dp::issue(st, i + NSLOT - 1, dslot(i + NSLOT - 1), wave, lane); };
        if constexpr (NPAR == 2) {
          refill();
          const int s = 2 * i + par;
          if (s < nslab) compute_slab<D>(p, it, s, dview(i, par), qf, kept, lim, ua, a_lo, c, m, l, o);
        } else {
          compute_pair<D>(p, it, 2 * i, nslab, dview(i, 0), dview(i, 1), qf, kept, lim, ua, a_lo, c, m, l, o,
                          refill);
        }
      }
      wait_vmcnt<0>();
      block_barrier();  // every copy has landed and every wave is done with the ring
    }
  }

  if constexpr (NPAR == 1) {
    if (!row_ok) return;
  } else {
    // ---- merge the two key parities of each row group through LDS (the ring
    //      is free after the loop's last barrier)
    float* mrg = (float*)ring;  // [RG row groups][D + 2][32]
    auto at = [&](int g, int d, int r) -> float& { return mrg[((size_t)g * (D + 2) + d) * 32 + r]; };
    if (npairs == 0) __syncthreads();
    if (par == 1) {
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) at(rg, head_dim(r, j, h), r32) = o[j][r];
      if (h == 0) { at(rg, D, r32) = m; at(rg, D + 1, r32) = l; }
    }
    __syncthreads();
    if (par == 1 || !row_ok) return;
    const float m1 = at(rg, D, r32), l1 = at(rg, D + 1, r32);
    const float mn = fmaxf(m, m1);
    const float mu = mn == -INFINITY ? 0.f : mn;
    const float a0 = __builtin_amdgcn_exp2f((m - mu) * c), a1 = __builtin_amdgcn_exp2f((m1 - mu) * c);
    l = l * a0 + l1 * a1;
    m = mn;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[j][r] = o[j][r] * a0 + at(rg, head_dim(r, j, h), r32) * a1;
  }
  const float inv = (kept && l > 0.f) ? 1.f / l : 0.f;
  uint16_t* orow = p.out + qrow * D;
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int qd = 0; qd < 4; ++qd)  // head dims 32j + 8qd + 4h .. +3
      *(u32x2*)(orow + head_dim(4 * qd, j, h)) =
          u32x2{pack_bf16x2(o[j][4 * qd] * inv, o[j][4 * qd + 1] * inv),
                pack_bf16x2(o[j][4 * qd + 2] * inv, o[j][4 * qd + 3] * inv)};
  if (p.lse && h == 0) {
    const int64_t li = ((int64_t)b * p.Hq + qh) * ((int64_t)p.A * p.gamma) + (int64_t)ua * p.gamma + uk;
    p.lse[li] = (kept && l > 0.f) ? m * p.scale + kLn2 * __builtin_amdgcn_logf(l) : -INFINITY;
  }
}

// ------------------------------------------------------ vector-ALU kernel
// float32 inputs (and any input the MFMA path does not take): one wave per
// (b, a, query head).  The block's rows go in groups of eight; for each
// group the visible keys go in chunks of 64: the chunk's K and V rows are
// copied into LDS with coalesced loads (lanes along the head dim), then
// lane j takes key j's scores against the eight query rows, each row takes
// an online-softmax step (wave reductions), and P.V runs with lanes along
// the head dim.
constexpr int kValuRows = 8;
template <bool kBf16>
__global__ __launch_bounds__(64) void block_attn_valu(Params p, int D) {
  __shared__ __align__(16) float qs[kValuRows][128];
  __shared__ float ks[64][129];  // +1: lane j's reads of row j hit distinct banks
  __shared__ float vs[64][128];
  __shared__ __align__(16) float ps[kValuRows][64];
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
  const int nkeys = kept ? lim + p.gamma : 0;
  const int64_t own0 = (int64_t)b * p.A * p.gamma + (int64_t)a * p.gamma;
  // head-dim offset of key j's row (context keys first, then the block's own)
  auto key_off = [&](int j) -> int64_t {
    const int64_t row = j < lim ? (int64_t)c0 + j : own0 + (j - lim);
    return (row * p.Hkv + kvh) * D;
  };
  for (int k0 = 0; k0 < p.gamma; k0 += kValuRows) {
    const int nr = min(kValuRows, p.gamma - k0);
    __syncthreads();
    {
      // all the group's Q loads in flight before the first store
      float qv[kValuRows][2];
#pragma unroll
      for (int kr = 0; kr < kValuRows; ++kr) {
        const int64_t qrow = (own0 + k0 + min(kr, nr - 1)) * p.Hq + h;
#pragma unroll
        for (int e = 0; e < 2; ++e) qv[kr][e] = lane + 64 * e < D ? ld(p.q, qrow * D + lane + 64 * e) : 0.f;
      }
#pragma unroll
      for (int kr = 0; kr < kValuRows; ++kr)
#pragma unroll
        for (int e = 0; e < 2; ++e)
          if (lane + 64 * e < D) qs[kr][lane + 64 * e] = qv[kr][e];
    }
    float m[kValuRows], l[kValuRows], o0[kValuRows], o1[kValuRows];
#pragma unroll
    for (int kr = 0; kr < kValuRows; ++kr) { m[kr] = -INFINITY; l[kr] = 0.f; o0[kr] = 0.f; o1[kr] = 0.f; }
    for (int j0 = 0; j0 < nkeys; j0 += 64) {
      const int nj = min(64, nkeys - j0);
      __syncthreads();  // the previous chunk's reads are done
      // eight keys' K and V loads in flight before their stores (one round
      // trip per eight keys, not per key)
      for (int jb = 0; jb < nj; jb += 8) {
        float kv[8][2], vv[8][2];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int jj = min(jb + u, nj - 1);
          const int64_t off = key_off(j0 + jj);
          const void* kp = j0 + jj < lim ? (const void*)p.kc : (const void*)p.kb;
          const void* vp = j0 + jj < lim ? (const void*)p.vc : (const void*)p.vb;
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int d = lane + 64 * e;
            kv[u][e] = d < D ? ld(kp, off + d) : 0.f;
            vv[u][e] = d < D ? ld(vp, off + d) : 0.f;
          }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (jb + u >= nj) break;
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int d = lane + 64 * e;
            if (d < D) {
              ks[jb + u][d] = kv[u][e];
              vs[jb + u][d] = vv[u][e];
            }
          }
        }
      }
      __syncthreads();
      // scores of key j0 + lane against the group's rows
      float sc[kValuRows];
#pragma unroll
      for (int kr = 0; kr < kValuRows; ++kr) sc[kr] = 0.f;
      if (lane < nj) {
        for (int d = 0; d < D; d += 4) {
          const float k0v = ks[lane][d], k1v = ks[lane][d + 1], k2v = ks[lane][d + 2], k3v = ks[lane][d + 3];
#pragma unroll
          for (int kr = 0; kr < kValuRows; ++kr) {
            const float4 q4 = *(const float4*)&qs[kr][d];
            sc[kr] = fmaf(q4.x, k0v, fmaf(q4.y, k1v, fmaf(q4.z, k2v, fmaf(q4.w, k3v, sc[kr]))));
          }
        }
      }
#pragma unroll
      for (int kr = 0; kr < kValuRows; ++kr) {
        const float s = lane < nj ? sc[kr] : -INFINITY;
        float smax = s;
        for (int off = 32; off > 0; off >>= 1) smax = fmaxf(smax, __shfl_xor(smax, off, 64));
        const float mn = fmaxf(m[kr], smax);
        const float mu = mn == -INFINITY ? 0.f : mn;
        const float alpha = __builtin_amdgcn_exp2f((m[kr] - mu) * c);
        const float pj = lane < nj ? __builtin_amdgcn_exp2f((s - mu) * c) : 0.f;
        float psum = pj;
        for (int off = 32; off > 0; off >>= 1) psum += __shfl_xor(psum, off, 64);
        l[kr] = l[kr] * alpha + psum;
        m[kr] = mn;
        o0[kr] *= alpha;
        o1[kr] *= alpha;
        ps[kr][lane] = pj;
      }
      __syncthreads();
      // P.V with lanes along the head dim
      for (int jj = 0; jj < nj; jj += 4) {
        float v0[4], v1[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          v0[t] = (jj + t < nj && lane < D) ? vs[jj + t][lane] : 0.f;
          v1[t] = (jj + t < nj && lane + 64 < D) ? vs[jj + t][lane + 64] : 0.f;
        }
#pragma unroll
        for (int kr = 0; kr < kValuRows; ++kr) {
          const float4 w = *(const float4*)&ps[kr][jj];  // entries past nj are zero
          o0[kr] = fmaf(w.x, v0[0], fmaf(w.y, v0[1], fmaf(w.z, v0[2], fmaf(w.w, v0[3], o0[kr]))));
          o1[kr] = fmaf(w.x, v1[0], fmaf(w.y, v1[1], fmaf(w.z, v1[2], fmaf(w.w, v1[3], o1[kr]))));
        }
      }
    }
#pragma unroll
    for (int kr = 0; kr < kValuRows; ++kr) {
      if (kr >= nr) break;
      const int k = k0 + kr;
      const int64_t qrow = (own0 + k) * p.Hq + h;
      const float inv = (kept && l[kr] > 0.f) ? 1.f / l[kr] : 0.f;
      if (kBf16) {
        uint16_t* o = (uint16_t*)p.out + qrow * D;
        if (lane < D) o[lane] = (uint16_t)f32_to_bf16(o0[kr] * inv);
        if (lane + 64 < D) o[lane + 64] = (uint16_t)f32_to_bf16(o1[kr] * inv);
      } else {
        float* o = (float*)p.out + qrow * D;
        if (lane < D) o[lane] = o0[kr] * inv;
        if (lane + 64 < D) o[lane + 64] = o1[kr] * inv;
      }
      if (p.lse && lane == 0) {
        const int64_t li = ((int64_t)b * p.Hq + h) * ((int64_t)p.A * p.gamma) + (int64_t)a * p.gamma + k;
        p.lse[li] = (kept && l[kr] > 0.f) ? m[kr] * p.scale + kLn2 * __builtin_amdgcn_logf(l[kr]) : -INFINITY;
      }
    }
  }
}

struct Shape {
  int group, ntiles, nrows;
  int64_t tiles;  // B * ntiles * Hkv
};

Shape make_shape(int B, int A, int gamma, int Hq, int Hkv, int rows = kTileRows) {
  Shape s{};
  s.group = Hq / Hkv;
  s.nrows = A * s.group * gamma;
  s.ntiles = (s.nrows + rows - 1) / rows;
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
  // a context read by at most two 64-row tiles per KV head streams from HBM
  // (64-row tiles, two load sets in flight); otherwise tiles of 128 rows
  // halve the K/V traffic per product
  const bool deep = make_shape(B, A, gamma, Hq, Hkv).ntiles <= 2;
  const int rows = deep ? 64 : 128;
  const Shape sh = make_shape(B, A, gamma, Hq, Hkv, rows);
  Params p{};
  p.q = (const uint16_t*)q; p.kc = (const uint16_t*)k_ctx; p.vc = (const uint16_t*)v_ctx;
  p.offs = ctx_offsets; p.kb = (const uint16_t*)k_blk; p.vb = (const uint16_t*)v_blk;
  p.anchor = anchor_pos; p.keep = keep_mask; p.out = (uint16_t*)out; p.lse = lse;
  p.status = dev_status;
  p.B = B; p.A = A; p.gamma = gamma; p.Hq = Hq; p.Hkv = Hkv; p.group = sh.group;
  p.ntiles = sh.ntiles; p.nrows = sh.nrows; p.tile_rows = rows; p.total_ctx = total_ctx; p.max_ctx = max_ctx;
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
    const dim3 grid((unsigned)sh.tiles), block(256);
    if (D == 128) {
      if (deep) hipLaunchKernelGGL((block_attn_mfma<128, 2, 2, 2>), grid, block, 0, s, p);
      else hipLaunchKernelGGL((block_attn_mfma<128, 4, 2, 1>), grid, block, 0, s, p);
    } else {
      if (deep) hipLaunchKernelGGL((block_attn_mfma<64, 2, 2, 2>), grid, block, 0, s, p);
      else hipLaunchKernelGGL((block_attn_mfma<64, 4, 2, 1>), grid, block, 0, s, p);
    }
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
