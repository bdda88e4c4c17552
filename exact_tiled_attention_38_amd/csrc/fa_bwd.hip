// Exact attention backward with recomputation, bf16 in/out, fp32 accumulation, gfx950.
//
// The method ("Attention and KV Compression", section "Recomputation in the
// backward pass"; "FlashAttention — how 100K-token attention fits in memory",
// section "Training backward"): the probabilities are not stored by the
// forward; every (query tile, key tile) pair recomputes S = scale Q K^T and
// P = exp(S - lse) from Q, K and the saved per-row logsumexp, then
//     dV += P^T dO,  dP = dO V^T,  dS = P * (dP - D),  D = rowsum(dO * O),
//     dK += scale dS^T Q,  dQ += scale dS K
// (the gradient of softmax attention; the pages give no formula, this is the
// derivative of the score/softmax/weight definition).
//
// Three kernels on the caller's stream:
//   1. preprocess: D_i = sum_k dO_ik O_ik and lse_i * log2(e) (fp32), into
//      the caller's workspace.
//   2. dkdv (this file): one workgroup per block of 128 keys of one key/value
//      head, 4 waves x 32 keys; with shared key/value heads it streams the
//      query tiles of every query head of its group in turn and sums their
//      contributions in the same registers. K and V rows of the wave stay in registers (the B
//      operands of S = Q K^T and dP = dO V^T); the fp32 dK^T and dV^T
//      accumulators stay in registers for the whole key block. Query tiles
//      of 64 rows (Q, dO, lse, D) arrive by direct-to-LDS loads into a
//      two-slot ring, one tile ahead. In this orientation each lane owns one
//      key and 16 of every 32 queries, so P and dS feed the dV^T = dO^T P and
//      dK^T = Q^T dS products straight from registers, with dO^T and Q^T
//      read from the row-major LDS tiles by ds_read_b64_tr_b16. Causal: query
//      tiles that end before the key block starts are never visited.
//   3. dq (fa_bwd_dq.hip): one workgroup per block of query rows streams the
//      key/value tiles and sums its rows' dQ itself, with no atomics.
// dq, dk and dv are all bitwise deterministic.
#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

// 1: the dP products start from D and V is negated, so the softmax gradient
// needs no subtraction per score
#ifndef FA_BWD_DFOLD
#define FA_BWD_DFOLD 1
#endif

constexpr int kBwdWaves = 4;
constexpr int kBwdKeys = 32 * kBwdWaves;  // keys per workgroup
constexpr int kBwdRows = 64;              // query rows per tile

// The dK/dV grid walks key/value heads in chunks of this many (one per XCD).
constexpr int kBwdHeadChunk = 8;

// Q and dO tiles (kBwdRows rows) arrive by direct-to-LDS loads into a
// two-slot ring, unpadded, with the 16-byte chunks of each row XOR-swizzled
// so that both the 128-bit row reads (16 rows, one chunk column) and the
// transposed reads (4 rows x 64 bytes) are free of bank conflicts.
template <int D> struct BwdCfg {
  static constexpr int ROWB = 2 * D;                      // Q/dO tile row bytes
  static constexpr int TILEB = kBwdRows * ROWB;           // one Q (or dO) tile
  static constexpr int CPR = D / 8;                       // 16-byte chunks per row
  static constexpr int RPW = 1024 / ROWB;                 // rows per wave-wide 1 KB load
  static constexpr int NDMA = TILEB / 1024 / kBwdWaves;   // wave-wide loads per wave and tensor
  static_assert(TILEB % (1024 * kBwdWaves) == 0, "tile must split into whole wave-wide loads");
};

// Chunk swizzle of the Q/dO tiles. D = 128 (one row per 256-byte bank
// line): bits 3..2 come from row bits 1..0 (the 4 rows of a transposed read
// land in distinct 64-byte quarters), bits 1..0 from row bits 3..2 (16
// consecutive rows get 16 distinct chunks). D = 64 (two rows per line): the
// same with row bits 1 and 3..2, as row bit 0 already selects the half line.
template <int D>
__device__ __forceinline__ int qswz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// ---------------------------------------------------------------- preprocess

template <int D>
__global__ void __launch_bounds__(256)
bwd_preprocess_kernel(const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO,
                      const float* __restrict__ LSE, float* __restrict__ Dvec,
                      float* __restrict__ L2vec, long long rows) {
  constexpr int LPR = D / 8;  // lanes per row, 8 elements each
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long row = gid / LPR;
  const int sub = (int)(gid % LPR);
  float sum = 0.f;
  if (row < rows) {
    const size_t off = (size_t)row * D + sub * 8;
    const bf16x8_t o = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(O + off));
    const bf16x8_t g = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(dO + off));
#pragma unroll
    for (int e = 0; e < 8; ++e) sum = fmaf((float)o[e], (float)g[e], sum);
  }
#pragma unroll
  for (int x = LPR / 2; x >= 1; x >>= 1) sum += __shfl_xor(sum, x, LPR);
  if (row < rows && sub == 0) {
    Dvec[row] = sum;
    L2vec[row] = LSE[row] * kLog2e;  // the dK/dV kernel's exponent offset, base 2
  }
}

// ---------------------------------------------------------------- dK / dV

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(64 * kBwdWaves, 1)
bwd_dkdv_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                const float* __restrict__ L2vec, const float* __restrict__ Dvec,
                uint16_t* __restrict__ dK, uint16_t* __restrict__ dV,
                int N, int n_kblocks, int n_kvheads, int group, float c2, float scale) {
  using C = BwdCfg<D>;
  // ring slot s: Q tile at qd + (2s) TILEB, dO tile at qd + (2s+1) TILEB
  __shared__ __attribute__((aligned(1024))) char qd[4 * C::TILEB];
  __shared__ __attribute__((aligned(16))) float rowstat[2][2][kBwdRows];  // [slot][lse, D][row]
  FA_LDS char* qdl = (FA_LDS char*)qd;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, n = lane & 31;
  // workgroup -> (key/value head, key block); the key/value head is shared
  // by query heads kvbh * group .. + group - 1, whose gradients it sums.
  // The grid takes the heads in chunks of kBwdHeadChunk and, inside a chunk,
  // goes key-block-major: workgroup b runs on XCD b % 8, so each XCD keeps
  // to one head of the chunk and its concurrent key blocks share that head's
  // query tiles in L2, and under a causal mask the longest key blocks (the
  // first ones) start first, so the last workgroups to start are short.
  const int chunk = blockIdx.x / (kBwdHeadChunk * n_kblocks);
  const int r = blockIdx.x - chunk * (kBwdHeadChunk * n_kblocks);
  const int cc = min(kBwdHeadChunk, n_kvheads - kBwdHeadChunk * chunk);  // heads in this chunk
  const int kbi = r / cc;
  const int kvbh = __builtin_amdgcn_readfirstlane(kBwdHeadChunk * chunk + r - kbi * cc);
  const int kb0 = __builtin_amdgcn_readfirstlane(kbi * kBwdKeys);
  const int kw0 = kb0 + 32 * w;
  const int key = kw0 + n;
  const size_t head = (size_t)kvbh * N * D;
  // the query head being streamed (set per head of the group below)
  int bh = 0;
  const uint16_t* Qh = Q;
  const uint16_t* dOh = dO;

  // this lane's key and value row as MFMA B operands: K[key][16c + 8h .. +7]
  bf16x8_t kf[D / 16], vf[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    u32x4_t a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
    if (key < N) {
      a = *(const u32x4_t*)(K + head + (size_t)key * D + 16 * c + 8 * h);
      b = *(const u32x4_t*)(V + head + (size_t)key * D + 16 * c + 8 * h);
    }
    kf[c] = __builtin_bit_cast(bf16x8_t, a);
    vf[c] = __builtin_bit_cast(bf16x8_t, b);
  }
  // take delivery of these loads before the tile loads start (they are not
  // counted by the explicit waits below)
#pragma unroll
  for (int c = 0; c < D / 16; ++c) asm volatile("" :: "v"(kf[c]), "v"(vf[c]));
  __builtin_amdgcn_s_waitcnt(0);
#if FA_BWD_DFOLD
  // V enters dP only: negated once here (bf16 sign bits), the dP products
  // start from the rows' D and so yield D - dP directly (see grad_pair)
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    u32x4_t x = __builtin_bit_cast(u32x4_t, vf[c]);
    x ^= 0x80008000u;
    vf[c] = __builtin_bit_cast(bf16x8_t, x);
  }
#endif

  f32x16_t dvacc[D / 32], dkacc[D / 32];
#pragma unroll
  for (int j = 0; j < D / 32; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) { dvacc[j][i] = 0.f; dkacc[j][i] = 0.f; }

  // ---- tile loads: wave w fills 1 KB blocks w*NDMA .. of the Q and dO tiles
  uint32_t qd_off[C::NDMA];
#pragma unroll
  for (int i = 0; i < C::NDMA; ++i) {
    const int r = (w * C::NDMA + i) * C::RPW + lane / C::CPR;
    qd_off[i] = r * C::ROWB + 16 * ((lane % C::CPR) ^ qswz<D>(r));
  }
  auto load_tile = [&](int q0, int slot) {
    const char* qb = (const char*)(Qh + (size_t)q0 * D);
    const char* gb = (const char*)(dOh + (size_t)q0 * D);
    FA_LDS char* dq_ = qdl + (2 * slot) * C::TILEB + w * C::NDMA * 1024;
    FA_LDS char* dg_ = qdl + (2 * slot + 1) * C::TILEB + w * C::NDMA * 1024;
    if (q0 + kBwdRows <= N) {
#pragma unroll
      for (int i = 0; i < C::NDMA; ++i) {
        dma16(qb, qd_off[i], dq_ + i * 1024);
        dma16(gb, qd_off[i], dg_ + i * 1024);
      }
    } else {
      // rows past N are fetched from row N-1 (finite) and masked below
      const int lim = N - 1 - q0;
#pragma unroll
      for (int i = 0; i < C::NDMA; ++i) {
        const uint32_t off = (uint32_t)min((int)(qd_off[i] / C::ROWB), lim) * C::ROWB + qd_off[i] % C::ROWB;
        dma16(qb, off, dq_ + i * 1024);
        dma16(gb, off, dg_ + i * 1024);
      }
    }
    if (w < 2) {  // wave 0: the rows' lse * log2(e), wave 1: their D
      const char* src = (const char*)((w == 0 ? L2vec : Dvec) + (size_t)bh * N + q0);
      dma4(src, 4u * (uint32_t)min(lane, N - 1 - q0), (FA_LDS char*)&rowstat[slot][w][0]);
    }
  };

  // LDS read offsets within a tile (bytes). Row reads (A operand rows of S
  // and dP): row n (+32 qb), logical chunk 2c + h, at row_off ^ (32 c).
  const int row_off = n * C::ROWB + 16 * (h ^ qswz<D>(n));
  // Transposed reads (dO^T, Q^T): rows 4h + q (+16 jj, +32 qb) and 8 more,
  // columns 32 j + 16 x + 4 (lane & 3), at tr_off[hi] ^ (64 j).
  const int tr_row = 4 * h + ((lane >> 2) & 3);
  const int tr_chunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int tr_off0 = tr_row * C::ROWB + 16 * (tr_chunk ^ qswz<D>(tr_row)) + 8 * (lane & 1);
  const int tr_off1 = (tr_row + 8) * C::ROWB + 16 * (tr_chunk ^ qswz<D>(tr_row + 8)) + 8 * (lane & 1);

  const int n_qtiles = (N + kBwdRows - 1) / kBwdRows;
  const int t_first = CAUSAL ? kb0 / kBwdRows : 0;
  const bool keys_tail = kb0 + kBwdKeys > N;


  // One query tile. MASKED: the tile has invisible (query, key) pairs (a key
  // after a query, a key past N, or a query row past N) and its scores are
  // masked; the other tiles run without any mask code.
  auto tile = [&](int t, auto masked) {
    constexpr bool need_mask = decltype(masked)::value;
    const int q0 = t * kBwdRows;
    const int slot = (t - t_first) & 1;
    if (t + 1 < n_qtiles) load_tile(q0 + kBwdRows, slot ^ 1);
    const FA_LDS char* Qs = qdl + (2 * slot) * C::TILEB;
    const FA_LDS char* Gs = qdl + (2 * slot + 1) * C::TILEB;
    // (the base offsets pass through an empty asm statement once per tile so
    // the compiler forms the per-chunk XORs here instead of keeping them all
    // live across the loop)
    int ro = row_off, to0 = tr_off0, to1 = tr_off1;
    asm volatile("" : "+v"(ro), "+v"(to0), "+v"(to1));

    // The tile as an explicit schedule of four phases over its two 32-row
    // query blocks (waves whose keys all follow the tile's queries run it
    // too, fully masked: P = dS = 0, which keeps one straight path):
    //   A0: S(0), dP(0)                                 matrix
    //   A1: S(1), dP(1)  with 6 of the 8 pairs of P/dS(0) matrix + vector
    //   B0: dV, dK(0)    with the rest of P/dS(0), then
    //                    the first half of P/dS(1)        matrix + vector
    //   B1: dV, dK(1)    with the second half of P/dS(1)  matrix + vector
    // (each half of a block's P/dS is complete before the first slice that
    // multiplies it; spreading it this way keeps any phase from carrying
    // more vector work than its matrix instructions can cover)
    // Each matrix instruction closes a scheduling slice; its LDS reads are
    // issued two slices ahead. S and dP: lane holds key `key`, queries
    // qb*32 + 8(i/4) + 4h + i%4.
    constexpr int NC = D / 16;       // S/dP slices per query block
    constexpr int NB = 2 * (D / 32); // dV/dK slices per query block (jj, j)
    // gradient pairs of block 0 moved from A1 into the first slices of B0
    constexpr int K0 = 2;
    static_assert(K0 <= NB / 2 && K0 < NB, "block 0 must be complete before B0 uses its second half");
    auto rread = [&](const FA_LDS char* base, int qb, int c) {
      return *(const FA_LDS bf16x8_t*)(base + qb * 32 * C::ROWB + (ro ^ (32 * c)));
    };
    auto tread = [&](const FA_LDS char* base, int qb, int m) {
      const int jj = m / (D / 32), j = m % (D / 32);
      const int rb = (qb * 32 + 16 * jj) * C::ROWB;
      return concat8(lds_read_tr4(base + rb + (to0 ^ (64 * j))), lds_read_tr4(base + rb + (to1 ^ (64 * j))));
    };
    f32x16_t s[2], dp[2];
    bf16x8_t pb[2][2], dsb[2][2];
    // the rows' lse * log2(e) and D for block qb, read from the tile's row
    // statistics one phase before their use (lane's rows 8g + 4h .. + 3)
    f32x4_t st_l[2][4], st_d[2][4];
    auto read_stats = [&](int qb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        st_l[qb][g] = *(const FA_LDS f32x4_t*)&rowstat[slot][0][qb * 32 + 8 * g + 4 * h];
        st_d[qb][g] = *(const FA_LDS f32x4_t*)&rowstat[slot][1][qb * 32 + 8 * g + 4 * h];
      }
    };
    // the accumulator a dP product chain starts from: the rows' D in the
    // accumulator's layout (element i: row 8(i/4) + 4h + i%4), or 0
    auto dinit = [&](int qb) {
      f32x16_t r = {};
#if FA_BWD_DFOLD
#pragma unroll
      for (int i = 0; i < 16; ++i) r[i] = st_d[qb][i >> 2][i & 3];
#endif
      return r;
    };
    // P and dS (bf16) for elements 2pr, 2pr+1 of block qb
    auto grad_pair = [&](int qb, int pr) {
      const int i = 2 * pr, g = i >> 2, e = i & 3;
      const float p0 = exp2_fast(fmaf(s[qb][i], c2, -st_l[qb][g][e]));
      const float p1 = exp2_fast(fmaf(s[qb][i + 1], c2, -st_l[qb][g][e + 1]));
      const bf16x2_t pp = to_bf16x2(p0, p1);
#if FA_BWD_DFOLD
      // dp holds D - dP: dS = P (dP - D) = -P (D - dP)
      const bf16x2_t dd = to_bf16x2(p0 * -dp[qb][i], p1 * -dp[qb][i + 1]);
#else
      const bf16x2_t dd = to_bf16x2(p0 * (dp[qb][i] - st_d[qb][g][e]), p1 * (dp[qb][i + 1] - st_d[qb][g][e + 1]));
#endif
      pb[qb][i >> 3][i & 7] = pp[0];
      pb[qb][i >> 3][(i & 7) + 1] = pp[1];
      dsb[qb][i >> 3][i & 7] = dd[0];
      dsb[qb][i >> 3][(i & 7) + 1] = dd[1];
    };
    // causal / tail mask of block qb: scores of invisible pairs -> -inf
    auto mask = [&](int qb) {
      // visible queries of this lane's key: qlo <= q < qhi
      const int qlo = (CAUSAL ? key : 0) - q0 - qb * 32 - 4 * h;
      const int qhi = (key < N ? N : 0) - q0 - qb * 32 - 4 * h;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int qo = 8 * (i >> 2) + (i & 3);
        if (qo < qlo || qo >= qhi) s[qb][i] = -INFINITY;
      }
    };

    bf16x8_t ra[NC], rg[NC];
    read_stats(0);
#if FA_BWD_DFOLD
    read_stats(1);  // (block 1's D seeds its dP products in A1)
#endif
    ra[0] = rread(Qs, 0, 0); rg[0] = rread(Gs, 0, 0);
    ra[1] = rread(Qs, 0, 1); rg[1] = rread(Gs, 0, 1);
    __builtin_amdgcn_sched_barrier(0);
    // A0
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int cn = c + 2;  // read two slices ahead (into block 1 at the end)
      if (cn < NC) { ra[cn] = rread(Qs, 0, cn); rg[cn] = rread(Gs, 0, cn); }
      else { ra[cn - NC] = rread(Qs, 1, cn - NC); rg[cn - NC] = rread(Gs, 1, cn - NC); }
      const f32x16_t z = {};
      s[0] = mfma_32x32x16(ra[c], kf[c], c == 0 ? z : s[0]);
      dp[0] = mfma_32x32x16(rg[c], vf[c], c == 0 ? dinit(0) : dp[0]);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (need_mask) mask(0);
    // A1 with the softmax gradient of block 0
#if !FA_BWD_DFOLD
    read_stats(1);
#endif
    bf16x8_t ta[NB], tg[NB];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int cn = c + 2;
      if (cn < NC) { ra[cn] = rread(Qs, 1, cn); rg[cn] = rread(Gs, 1, cn); }
      else { ta[cn - NC] = tread(Qs, 0, cn - NC); tg[cn - NC] = tread(Gs, 0, cn - NC); }
      const f32x16_t z = {};
      s[1] = mfma_32x32x16(ra[c], kf[c], c == 0 ? z : s[1]);
      dp[1] = mfma_32x32x16(rg[c], vf[c], c == 0 ? dinit(1) : dp[1]);
#pragma unroll
      for (int pr = c * (8 - K0) / NC; pr < (c + 1) * (8 - K0) / NC; ++pr) grad_pair(0, pr);
      __builtin_amdgcn_sched_barrier(0);
    }
    // (the first half of block 0's P and dS is complete here: keep the
    // compiler from sinking it past the branch below, away from these
    // matrix instructions)
    asm volatile("" :: "v"(pb[0][0]), "v"(dsb[0][0]));
    if constexpr (need_mask) mask(1);
    // B0 (dV^T += dO^T P, dK^T += Q^T dS over block 0) with block 1's gradient
#pragma unroll
    for (int m = 0; m < NB; ++m) {
      const int mn = m + 2;
      if (mn < NB) { ta[mn] = tread(Qs, 0, mn); tg[mn] = tread(Gs, 0, mn); }
      else { ta[mn - NB] = tread(Qs, 1, mn - NB); tg[mn - NB] = tread(Gs, 1, mn - NB); }
      const int jj = m / (D / 32), j = m % (D / 32);
      // block 0's last K0 pairs first (its second half is used from slice
      // NB/2 on), then the first half of block 1 (used in B1)
      if (m < K0) grad_pair(0, 8 - K0 + m);
      else {
#pragma unroll
        for (int pr = (m - K0) * 4 / (NB - K0); pr < (m - K0 + 1) * 4 / (NB - K0); ++pr) grad_pair(1, pr);
      }
      dvacc[j] = mfma_32x32x16(tg[m], pb[0][jj], dvacc[j]);
      dkacc[j] = mfma_32x32x16(ta[m], dsb[0][jj], dkacc[j]);
      __builtin_amdgcn_sched_barrier(0);
    }
    asm volatile("" :: "v"(pb[1][0]), "v"(dsb[1][0]));
    // B1
#pragma unroll
    for (int m = 0; m < NB; ++m) {
      const int mn = m + 2;
      if (mn < NB) { ta[mn] = tread(Qs, 1, mn); tg[mn] = tread(Gs, 1, mn); }
      const int jj = m / (D / 32), j = m % (D / 32);
      // the second half of block 1, used from slice NB/2 on
      if (m < NB / 2) {
#pragma unroll
        for (int pr = 4 + m * 8 / NB; pr < 4 + (m + 1) * 8 / NB; ++pr) grad_pair(1, pr);
      }
      dvacc[j] = mfma_32x32x16(tg[m], pb[1][jj], dvacc[j]);
      dkacc[j] = mfma_32x32x16(ta[m], dsb[1][jj], dkacc[j]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // the next tile's Q/dO/lse/D have landed; this tile's slot is free
    wait_loads_and_barrier<0>();
  };

  // Tiles in three runs so the common one has no mask code at all: the
  // diagonal tiles (causal: those starting before the key block's last key),
  // the interior tiles, then a ragged last tile. A key block reaching past N
  // masks every tile.
  const int t_inner = keys_tail ? n_qtiles
                                : min(n_qtiles, CAUSAL ? (kb0 + kBwdKeys - 1) / kBwdRows + 1 : 0);
  const int t_tail = keys_tail ? n_qtiles : (N / kBwdRows);  // first tile with rows past N
  for (int g = 0; g < group; ++g) {
    bh = __builtin_amdgcn_readfirstlane(kvbh * group + g);
    Qh = Q + (size_t)bh * N * D;
    dOh = dO + (size_t)bh * N * D;
    // (every wave is past the previous head's last tile: its closing
    // barrier has run, so slot 0 is free)
    load_tile(t_first * kBwdRows, 0);
    wait_loads_and_barrier<0>();
    int t = t_first;
    for (; t < t_inner; ++t) tile(t, std::true_type{});
    for (; t < t_tail; ++t) tile(t, std::false_type{});
    for (; t < n_qtiles; ++t) tile(t, std::true_type{});
  }

  // dK = scale * (dK^T)^T, dV = (dV^T)^T: lane holds its key's d values in groups of 4
  if (key < N) {
#pragma unroll
    for (int j = 0; j < D / 32; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * j + 8 * g + 4 * h;
        const bf16x2_t k01 = to_bf16x2(scale * dkacc[j][4 * g], scale * dkacc[j][4 * g + 1]);
        const bf16x2_t k23 = to_bf16x2(scale * dkacc[j][4 * g + 2], scale * dkacc[j][4 * g + 3]);
        const bf16x2_t v01 = to_bf16x2(dvacc[j][4 * g], dvacc[j][4 * g + 1]);
        const bf16x2_t v23 = to_bf16x2(dvacc[j][4 * g + 2], dvacc[j][4 * g + 3]);
        const u32x2_t kk = {__builtin_bit_cast(uint32_t, k01), __builtin_bit_cast(uint32_t, k23)};
        const u32x2_t vv = {__builtin_bit_cast(uint32_t, v01), __builtin_bit_cast(uint32_t, v23)};
        *(u32x2_t*)(dK + head + (size_t)key * D + d0) = kk;
        *(u32x2_t*)(dV + head + (size_t)key * D + d0) = vv;
      }
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const void* q, const void* k, const void* v, const void* o, const void* dO,
                  const float* lse, void* dq, void* dk, void* dv, void* workspace, const Problem& p,
                  hipStream_t stream) {
  const long long rows = (long long)p.B * p.H * p.N;
  float* Dvec = (float*)workspace;  // [B, H, N] D, then [B, H, N] lse * log2(e)
  float* L2vec = Dvec + rows;
  {
    const long long threads = rows * (D / 8);
    const long long blocks = (threads + 255) / 256;
    hipLaunchKernelGGL(bwd_preprocess_kernel<D>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const uint16_t*)o, (const uint16_t*)dO, lse, Dvec, L2vec, rows);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    const int n_kblocks = (p.N + kBwdKeys - 1) / kBwdKeys;
    const long long blocks = (long long)p.B * p.Hkv * n_kblocks;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3((unsigned)blocks), dim3(64 * kBwdWaves), 0,
                       stream, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                       (const uint16_t*)dO, (const float*)L2vec, (const float*)Dvec, (uint16_t*)dk, (uint16_t*)dv,
                       p.N, n_kblocks, p.B * p.Hkv, p.group(), p.scale * kLog2e, p.scale);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_bwd_dq(q, k, v, dO, lse, Dvec, dq, p, stream);
}

}  // namespace

hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const void* o,
                           const void* dO, const float* lse, void* dq, void* dk, void* dv,
                           void* workspace, const Problem& p, hipStream_t stream) {
  if (p.d == 128)
    return p.causal ? launch<128, true>(q, k, v, o, dO, lse, dq, dk, dv, workspace, p, stream)
                    : launch<128, false>(q, k, v, o, dO, lse, dq, dk, dv, workspace, p, stream);
  return p.causal ? launch<64, true>(q, k, v, o, dO, lse, dq, dk, dv, workspace, p, stream)
                  : launch<64, false>(q, k, v, o, dO, lse, dq, dk, dv, workspace, p, stream);
}

}  // namespace fa
