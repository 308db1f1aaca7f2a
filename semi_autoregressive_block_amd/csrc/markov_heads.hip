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
//   bf16 MFMA contraction over d: 128 x 128 output tiles, operands staged
//   in LDS by direct-to-LDS copies, v_mfma_f32_32x32x16_bf16, and the
//   contraction split over workgroups (partial tiles summed by the reader)
//   so that a few hundred workgroups fill the chip.
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
constexpr int kRowsPer = 16;    // rows per recurrent-step workgroup
constexpr int kChanPer = 8;     // channels per recurrent-step workgroup
constexpr int kMaxRank = 512;

// P_z[i][c] = sum_{k in split z} A[i][k] B[c][k] for i < M, c < N (bf16 in, float32 out): the
// hidden-state part of the heads' maps.  A rows are lda elements apart, B rows ldb; K, lda, ldb
// multiples of 8 and both bases 16-byte aligned (checked by the host).
//
// A workgroup of eight waves owns a 128 x 128 output tile and one contiguous split of the
// contraction (blockIdx.z; a second kernel sums the splits' partial tiles in fixed order, so
// results do not depend on scheduling).  The contraction goes in 64-wide slabs through a
// four-stage LDS ring filled by direct-to-LDS copies (three slabs, 96 KB, in flight; one
// workgroup per compute unit): a stage holds the tile's 128 A rows and 128 B rows, 128 bytes
// each, so every copy instruction fetches whole 128-byte lines.  The LDS serves a 16-byte read
// sixteen lanes (256 bytes) at a time, and a read instruction's lanes 0-15 take 16 consecutive
// rows, so piece p of row x is stored at p ^ ((x >> 1) & 7): rows x and x + 1 fall in the two
// halves of the banks and the eight pairs in distinct 16-byte bank groups.  Wave (wm, wn) computes
// the 64 x 32 piece at rows 64 wm, columns 32 wn as two products v_mfma_f32_32x32x16_bf16 with B
// as the first operand, so lane l ends up holding row l mod 32 of a product and columns
// 8q + 4(l / 32) .. +3: 16-byte stores.  Two waves per SIMD, because one wave alone cannot keep the
// LDS busy.  A stage's twelve operand reads per wave go out together, one stage ahead of the
// products (two register sets, used in turn), and they are inline assembly with the wait in a
// separate statement, because the compiler would otherwise wait for every copy in flight before
// each of them.
constexpr int kGemmTile = 128;
constexpr int kGemmSlab = 64;
constexpr int kGemmStages = 4;
constexpr int kGemmWaves = 8;
constexpr int kGemmPieces = kGemmSlab / 8;                  // 16-byte pieces of a row per slab
constexpr int kGemmRowBytes = kGemmSlab * 2;
constexpr int kGemmStageBytes = 2 * kGemmTile * kGemmRowBytes;  // A and B pieces of one slab
constexpr int kGemmCopies = kGemmStageBytes / 1024;             // 1 KB copies per stage
constexpr int kGemmCopiesPerWave = kGemmCopies / kGemmWaves;
static_assert(kGemmPieces == 8, "the bank swizzle below assumes 128-byte rows");

// Three 16-byte LDS reads, no wait: the results are not defined until lds_wait12 below.
__device__ __forceinline__ void lds_issue3_b128(uint32_t a0, uint32_t a1, uint32_t a2, u32x4& x0, u32x4& x1,
                                                u32x4& x2) {
  asm volatile("ds_read_b128 %0, %3\n\tds_read_b128 %1, %4\n\tds_read_b128 %2, %5"
               : "=&v"(x0), "=&v"(x1), "=&v"(x2)
               : "v"(a0), "v"(a1), "v"(a2)
               : "memory");
}
// Waits for every LDS read in flight; the registers the reads fill are defined again here, so no
// use of them moves above the wait.
__device__ __forceinline__ void lds_wait12(u32x4 (&r)[12]) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]), "+v"(r[4]), "+v"(r[5]), "+v"(r[6]), "+v"(r[7]),
                 "+v"(r[8]), "+v"(r[9]), "+v"(r[10]), "+v"(r[11])::"memory");
}

__device__ __forceinline__ void wait_vmcnt_copies(int n) {  // n = copies allowed in flight (a multiple of 4)
  switch (n) {
    case 0: wait_vmcnt<0>(); break;
    case 4: wait_vmcnt<4>(); break;
    case 8: wait_vmcnt<8>(); break;
    case 12: wait_vmcnt<12>(); break;
    default: wait_vmcnt<16>(); break;
  }
}
static_assert(kGemmCopiesPerWave * (kGemmStages - 2) <= 16 && kGemmCopiesPerWave % 4 == 0,
              "copies in flight beyond the waits above");

__global__ __launch_bounds__(64 * kGemmWaves) void head_proj_gemm(const uint16_t* __restrict__ A, int64_t lda,
                                                                  const uint16_t* __restrict__ B, int64_t ldb,
                                                                  float* __restrict__ P, int64_t split_stride,
                                                                  int M, int N, int K, int kchunk) {
  __shared__ __align__(16) unsigned char ring[kGemmStages * kGemmStageBytes];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave & 1, wn = wave >> 1;  // rows 64 wm, columns 32 wn of the tile
  const int i0 = blockIdx.x * kGemmTile, c0 = blockIdx.y * kGemmTile;
  const int kb = blockIdx.z * kchunk, ke = min(K, kb + kchunk);
  const int nst = (ke - kb + kGemmSlab - 1) / kGemmSlab;  // >= 1: the host launches no empty split

  // copies: per stage 32 of 1 KB (A then B), 4 per wave; copy c, lane l -> LDS chunk 64 c + l of the
  // stage = row x = (64 c + l) / 8 of A (c < 16) or B, stored piece (l & 7), which holds the row's
  // piece (l & 7) ^ ((x >> 1) & 7)
  constexpr int kHalf = kGemmCopies / 2;
  const uint16_t* src[kGemmCopiesPerWave];
  int kpiece[kGemmCopiesPerWave];
#pragma unroll
  for (int j = 0; j < kGemmCopiesPerWave; ++j) {
    const int c = wave * kGemmCopiesPerWave + j;  // 0 .. 31
    const int x = ((c % kHalf) * 64 + lane) / kGemmPieces;
    const int piece = (lane % kGemmPieces) ^ ((x >> 1) & 7);
    src[j] = c < kHalf ? A + (int64_t)min(i0 + x, M - 1) * lda : B + (int64_t)min(c0 + x, N - 1) * ldb;
    kpiece[j] = piece * 8;
  }
  auto issue = [&](int st) {
    unsigned char* dst = ring + (st % kGemmStages) * kGemmStageBytes;
    const int k = kb + st * kGemmSlab;
#pragma unroll
    for (int j = 0; j < kGemmCopiesPerWave; ++j) {
      // a piece past the contraction end reads the row's first piece (valid memory); its products
      // are dropped below by zeroing the operands
      const int kk = k + kpiece[j] < ke ? k + kpiece[j] : 0;
      __builtin_amdgcn_global_load_lds(
          (const void*)(src[j] + kk),
          (__attribute__((address_space(3))) void*)(dst + (wave * kGemmCopiesPerWave + j) * 1024), 16, 0, 0);
    }
  };

  f32x16 acc[2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[a][r] = 0.f;

  // this lane's operand rows: A rows 64 wm + 32 a + (l & 31), B row 32 wn + (l & 31); the piece of
  // k16 step t is 2 t + (l >> 5)
  const uint32_t ring_lds = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)ring;
  uint32_t roff[3];  // byte offsets of the three operand rows inside a stage
  int rsw[3];
#pragma unroll
  for (int q = 0; q < 3; ++q) {
    const int x = (q < 2 ? 64 * wm + 32 * q : 32 * wn) + (lane & 31);
    roff[q] = (uint32_t)((q < 2 ? 0 : kGemmTile * kGemmRowBytes) + x * kGemmRowBytes);
    rsw[q] = (x >> 1) & 7;
  }
  const int h = lane >> 5;

  const int pre = nst < kGemmStages - 1 ? nst : kGemmStages - 1;
  for (int st = 0; st < pre; ++st) issue(st);
  // stage st's copies are in (every wave's, after the barrier) and stage st - 1 is consumed: its
  // slot takes the copies of stage st + 3
  auto stage_in = [&](int st) {
    wait_vmcnt_copies(kGemmCopiesPerWave * min(nst - 1 - st, kGemmStages - 2));
    __builtin_amdgcn_s_barrier();
    if (st + kGemmStages - 1 < nst) issue(st + kGemmStages - 1);
  };
  auto read_stage = [&](int st, u32x4 (&r)[12]) {
    const uint32_t sbase = ring_lds + (st % kGemmStages) * kGemmStageBytes;
#pragma unroll
    for (int t = 0; t < kGemmSlab / 16; ++t) {
      const int pc = 2 * t + h;
      lds_issue3_b128(sbase + roff[0] + ((pc ^ rsw[0]) << 4), sbase + roff[1] + ((pc ^ rsw[1]) << 4),
                      sbase + roff[2] + ((pc ^ rsw[2]) << 4), r[3 * t], r[3 * t + 1], r[3 * t + 2]);
    }
  };
  auto products = [&](const u32x4 (&c)[12]) {
#pragma unroll
    for (int t = 0; t < kGemmSlab / 16; ++t) {
      acc[0] = mfma32x32x16(c[3 * t + 2], c[3 * t], acc[0]);
      acc[1] = mfma32x32x16(c[3 * t + 2], c[3 * t + 1], acc[1]);
    }
  };
  // stage st's products from registers c while stage st + 1's reads land in n
  auto body = [&](int st, const u32x4 (&c)[12], u32x4 (&n)[12]) {
    stage_in(st + 1);
    read_stage(st + 1, n);
    __builtin_amdgcn_sched_barrier(0);
    products(c);
    __builtin_amdgcn_sched_barrier(0);
    lds_wait12(n);
  };
  // the last stage: its pieces past the contraction end become zero
  auto last = [&](u32x4 (&c)[12]) {
    const int k = kb + (nst - 1) * kGemmSlab;
#pragma unroll
    for (int t = 0; t < kGemmSlab / 16; ++t)
      if (k + 8 * (2 * t + h) >= ke)
#pragma unroll
        for (int q = 0; q < 3; ++q) c[3 * t + q] = u32x4{0u, 0u, 0u, 0u};
    products(c);
  };
  // two register sets in turn (the loop takes stages in pairs, so neither is copied)
  u32x4 ra[12], rb[12];
  stage_in(0);
  read_stage(0, ra);
  lds_wait12(ra);
  int st = 0;
  for (; st + 2 < nst; st += 2) {
    body(st, ra, rb);
    body(st + 1, rb, ra);
  }
  if (st + 1 < nst) {
    body(st, ra, rb);
    last(rb);
  } else {
    last(ra);
  }

  // lane l: row i0 + 64 wm + 32 a + (l & 31), columns c0 + 32 wn + 8 q + 4 h .. +3 (N is a
  // multiple of 8, so a group that starts inside the row ends inside it)
  float* Pz = P + (int64_t)blockIdx.z * split_stride;
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int i = i0 + 64 * wm + 32 * a + (lane & 31);
    if (i >= M) continue;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = c0 + 32 * wn + 8 * q + 4 * h;
      if (c < N)
        *(f32x4*)(Pz + (int64_t)i * N + c) = f32x4{acc[a][4 * q], acc[a][4 * q + 1], acc[a][4 * q + 2], acc[a][4 * q + 3]};
    }
  }
}

// P[i] = sum_z P_z[i] in split order, for the n = M x N entries (16-byte vectors; n is a
// multiple of 8).
__global__ __launch_bounds__(256) void proj_sum_splits(float* __restrict__ P, int nsplit, int64_t n) {
  const int64_t v = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (v >= n) return;
  f32x4 acc = *(const f32x4*)(P + v);
  for (int z = 1; z < nsplit; ++z) acc += *(const f32x4*)(P + z * n + v);
  *(f32x4*)(P + v) = acc;
}

// Splits of the contraction for an M x N projection: at most one workgroup per compute unit of
// a 256-unit chip (the workgroup's LDS ring takes most of a unit), at most 8 splits.  Depends on
// M and N only, so the workspace can be sized without the contraction length.
int proj_splits(int M, int N) {
  const int64_t tiles = (int64_t)((M + kGemmTile - 1) / kGemmTile) * ((N + kGemmTile - 1) / kGemmTile);
  const int64_t sk = 256 / (tiles > 0 ? tiles : 1);
  return (int)(sk < 1 ? 1 : (sk > 8 ? 8 : sk));
}

template <bool kBf16>
__device__ __forceinline__ float ldw(const void* p, int64_t i) {
  return kBf16 ? __uint_as_float((uint32_t)((const uint16_t*)p)[i] << 16) : ((const float*)p)[i];
}

__device__ __forceinline__ float sigm(float x) { return 1.f / (1.f + expf(-x)); }

// One position of every row: rows row0 .. +15 and channels j0 .. +7 per
// workgroup; thread t takes (row i, channel jj) = ((t mod 128) / 8,
// t mod 8) and half kh = t / 128 of every chunk of the contraction, the two
// halves summed through LDS at the end.
//   z = [s; W1[x]] (RNN, length 2r) or W1[x] (gated, length r), in LDS
//   acc_q = W_q,rec[j] . z  (q = gate, candidate, output; or the gate alone)
// W_q,rec rows are ldwr elements apart, matrix q at wrec + q * mstride; the
// hidden-state part arrives in P[row, step, q * r + j].  The workgroup's
// weight rows are staged in LDS as float32 in 512-wide chunks of z, the next
// chunk's 16-byte loads in flight while the current chunk is used.  Rows
// are padded by 4 floats so that the rows a wave reads at one k fall in
// distinct LDS banks.  The first chunk and the hidden-state terms, which do
// not depend on the previous token, are loaded first.  The previous token
// is the caller's (prev_tok[row * prev_stride]) or the argmax folded in the
// previous step's keys.
constexpr int kChunk = 512;          // z entries per staged weight chunk
constexpr int kWPad = kChunk + 4;    // floats per staged weight row
__host__ __device__ constexpr size_t head_step_lds(bool rnn, int r) {
  return (size_t)(rnn ? 3 : 1) * kChanPer * kWPad * 4 + (size_t)kRowsPer * ((rnn ? 2 : 1) * r + 4) * 4 +
         kRowsPer * 4 + (size_t)(rnn ? 3 : 1) * 128 * 4;
}

template <bool RNN, bool kBf16W1>
__global__ __launch_bounds__(256) void head_step_kernel(
    const float* __restrict__ P, const void* __restrict__ w1, const uint16_t* __restrict__ wrec, int64_t ldwr,
    int64_t mstride, const int32_t* __restrict__ prev_tok, int64_t prev_stride,
    const uint64_t* __restrict__ keys_prev, const float* __restrict__ s_in, float* __restrict__ s_out,
    float* __restrict__ ebuf, int R, int gamma, int V, int r, int step, int32_t* __restrict__ status) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int NQ = RNN ? 3 : 1;
  const int zlen = RNN ? 2 * r : r, zst = zlen + 4;
  float* wl = (float*)smem;                          // [NQ][kChanPer][kWPad]
  float* z = wl + NQ * kChanPer * kWPad;             // [kRowsPer][zst]
  int* pv = (int*)(z + kRowsPer * zst);              // [kRowsPer]
  float* red = (float*)(pv + kRowsPer);              // [NQ][128]
  const int row0 = blockIdx.x * kRowsPer, j0 = blockIdx.y * kChanPer;
  const int t = threadIdx.x & 127, kh = threadIdx.x >> 7;
  const int i = t / kChanPer, jj = t % kChanPer, j = j0 + jj, row = row0 + i;
  // weight chunk c0: NQ x 8 rows of cw / 8 pieces, at most NQ per thread
  constexpr int kPer = NQ * kChanPer * (kChunk / 8) / 256;
  u32x4 wv[kPer];
  auto load_chunk = [&](int c0) {
    const int n8 = min(kChunk, zlen - c0) / 8, total = NQ * kChanPer * n8;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e = min((int)threadIdx.x + 256 * u, total - 1);
      const int q = e / (kChanPer * n8), rem = e % (kChanPer * n8), jr = rem / n8, k8 = rem % n8;
      wv[u] = *(const u32x4*)(wrec + q * mstride + (int64_t)min(j0 + jr, r - 1) * ldwr + c0 + 8 * k8);
    }
  };
  auto store_chunk = [&](int c0) {
    const int n8 = min(kChunk, zlen - c0) / 8, total = NQ * kChanPer * n8;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e = threadIdx.x + 256 * u;
      if (e < total) {
        const int q = e / (kChanPer * n8), rem = e % (kChanPer * n8), jr = rem / n8, k8 = rem % n8;
        float* dst = wl + (q * kChanPer + jr) * kWPad + 8 * k8;
        const u32x4 w = wv[u];
        *(f32x4*)dst = f32x4{bf16lo(w[0]), bf16hi(w[0]), bf16lo(w[1]), bf16hi(w[1])};
        *(f32x4*)(dst + 4) = f32x4{bf16lo(w[2]), bf16hi(w[2]), bf16lo(w[3]), bf16hi(w[3])};
      }
    }
  };
  load_chunk(0);
  const int64_t pos = (int64_t)min(row, R - 1) * gamma + step;
  float hp[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) hp[q] = P[pos * (NQ * r) + q * r + min(j, r - 1)];
  if (threadIdx.x < kRowsPer) {
    const int rw = row0 + threadIdx.x;
    int p = 0;
    if (rw < R) {
      p = keys_prev ? (int)argmax_key_index(read_key(keys_prev, rw, R)) : prev_tok[(int64_t)rw * prev_stride];
      if (p < 0 || p >= V) {
        if (blockIdx.y == 0) status_or(status, DSPARK_STATUS_BAD_TOKEN);
        p = 0;
      }
    }
    pv[threadIdx.x] = p;
  }
  __syncthreads();
  // z: 16-byte pieces from clamped, always-valid addresses (rows past R
  // read row R - 1 or token 0 and are never stored), in batches of 4 loads
  // per thread issued before any conversion or LDS store
  if constexpr (RNN) {
    const int n4 = r / 4, total = kRowsPer * n4;
    for (int c0 = threadIdx.x; c0 < total; c0 += 256 * 4) {
      f32x4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int cc = min(c0 + 256 * u, total - 1), rr = cc / n4, k4 = cc % n4;
        v[u] = *(const f32x4*)(s_in + (int64_t)min(row0 + rr, R - 1) * r + 4 * k4);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = c0 + 256 * u;
        if (c < total) *(f32x4*)(z + (c / n4) * zst + 4 * (c % n4)) = v[u];
      }
    }
  }
  {
    constexpr int per = kBf16W1 ? 8 : 4;  // W1 entries per 16-byte piece
    const int ne = r / per, total = kRowsPer * ne, eoff = RNN ? r : 0;
    for (int c0 = threadIdx.x; c0 < total; c0 += 256 * 4) {
      u32x4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int cc = min(c0 + 256 * u, total - 1), rr = cc / ne, kp = cc % ne;
        v[u] = *(const u32x4*)((const char*)w1 + ((int64_t)pv[rr] * r + (int64_t)kp * per) * (kBf16W1 ? 2 : 4));
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = c0 + 256 * u;
        if (c >= total) continue;
        float* dst = z + (c / ne) * zst + eoff + (c % ne) * per;
        if constexpr (kBf16W1) {
          *(f32x4*)dst = f32x4{bf16lo(v[u][0]), bf16hi(v[u][0]), bf16lo(v[u][1]), bf16hi(v[u][1])};
          *(f32x4*)(dst + 4) = f32x4{bf16lo(v[u][2]), bf16hi(v[u][2]), bf16lo(v[u][3]), bf16hi(v[u][3])};
        } else {
          *(f32x4*)dst = __builtin_bit_cast(f32x4, v[u]);
        }
      }
    }
  }
  float acc[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) acc[q] = 0.f;
  const float* zr = z + i * zst;
  for (int c0 = 0; c0 < zlen; c0 += kChunk) {
    const int cw = min(kChunk, zlen - c0);  // a multiple of 8: halves of multiples of 4
    __syncthreads();                        // z staged / previous chunk consumed
    store_chunk(c0);
    if (c0 + kChunk < zlen) load_chunk(c0 + kChunk);
    __syncthreads();
    const int k0 = kh * (cw / 2), k1 = k0 + cw / 2;
    for (int k = k0; k < k1; k += 4) {
      const f32x4 zv = *(const f32x4*)(zr + c0 + k);
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const f32x4 w = *(const f32x4*)(wl + (q * kChanPer + jj) * kWPad + k);
        float a = acc[q];
        a = fmaf(w[0], zv[0], a); a = fmaf(w[1], zv[1], a);
        a = fmaf(w[2], zv[2], a); a = fmaf(w[3], zv[3], a);
        acc[q] = a;
      }
    }
  }
  if (kh == 1) {
#pragma unroll
    for (int q = 0; q < NQ; ++q) red[q * 128 + t] = acc[q];
  }
  __syncthreads();
  if (kh == 1 || row >= R || j >= r) return;
#pragma unroll
  for (int q = 0; q < NQ; ++q) acc[q] += red[q * 128 + t];
  if constexpr (RNN) {
    const float gt = sigm(acc[0] + hp[0]);
    const float cand = tanhf(acc[1] + hp[1]);
    ebuf[pos * r + j] = tanhf(acc[2] + hp[2]);
    s_out[(int64_t)row * r + j] = gt * zr[j] + (1.f - gt) * cand;
  } else {
    ebuf[pos * r + j] = sigm(acc[0] + hp[0]) * zr[j];
  }
}

__global__ void fill_zero_f32(float* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Workspace layout: keys | P [splits][R*gamma, NQ*r] | E [R*gamma, r] | s ping-pong [2, R, r]
struct Layout {
  size_t keys, proj, emb, state, total;
};
Layout layout(int kind, int R, int gamma, int r, int64_t nkeys) {
  const int nq = kind == kHeadRnn ? 3 : 1;
  Layout L;
  L.keys = 0;
  L.proj = align256((size_t)nkeys * 8);
  L.emb = L.proj + align256((size_t)proj_splits(R * gamma, nq * r) * R * gamma * nq * r * 4);
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
  // contraction splits: partial tiles split_stride apart, then summed into the first
  const int sk_max = proj_splits(M, N);
  const int kchunk = ((a.d + sk_max - 1) / sk_max + kGemmSlab - 1) / kGemmSlab * kGemmSlab;
  const int nsplit = (a.d + kchunk - 1) / kchunk;  // <= sk_max, none empty
  const int64_t split_stride = (int64_t)M * N;
  hipLaunchKernelGGL(head_proj_gemm,
                     dim3((M + kGemmTile - 1) / kGemmTile, (N + kGemmTile - 1) / kGemmTile, nsplit),
                     dim3(64 * kGemmWaves), 0,
                     s, (const uint16_t*)a.hidden, (int64_t)a.d, Bh, ldw, P, split_stride, M, N, a.d, kchunk);
  if (nsplit > 1)
    hipLaunchKernelGGL(proj_sum_splits, dim3((unsigned)((split_stride / 4 + 255) / 256)), dim3(256), 0, s, P, nsplit,
                       split_stride);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (rnn) {
    const int64_t n = (int64_t)a.R * a.r;  // s_0 = 0
    hipLaunchKernelGGL(fill_zero_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, S, n);
  }
  const uint16_t* wrec = wh + (rnn ? 0 : a.d);
  const int64_t mstride = (int64_t)a.r * ldw;
  const size_t shm = head_step_lds(rnn, a.r);
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
  if ((uintptr_t)a.hidden % 16 || (uintptr_t)a.whead % 16 || (uintptr_t)a.w1 % 16)
    return fail(DSPARK_ERR_INVALID_ARG, "%s: hidden, w1 and head weights must be 16-byte aligned", what);
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
