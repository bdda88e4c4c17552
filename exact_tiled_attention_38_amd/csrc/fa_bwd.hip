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
//      head, 8 waves: each group of 32 keys is shared by two waves on one
//      SIMD, one for S, P and dV, the other (one query tile behind, with
//      its partner's P passed through LDS) for dP, dS and dK; with shared
//      key/value heads the query tiles of every query head of the group
//      form one stream, summed in the same registers. The wave's K or V rows
//      stay in registers (the B operands of S = Q K^T and dP = dO V^T), and
//      its fp32 dV^T or dK^T accumulator for the whole key block. Query
//      tiles of 64 rows (Q, dO, lse, D) arrive by direct-to-LDS loads into
//      a three-slot ring, one tile ahead. In this orientation each lane owns
//      one key and 16 of every 32 queries, so P and dS feed the
//      dV^T = dO^T P and dK^T = Q^T dS products straight from registers,
//      with dO^T and Q^T read from the row-major LDS tiles by
//      ds_read_b64_tr_b16. Causal: query tiles that end before the key
//      block starts are never visited.
//   3. dq (fa_bwd_dq.hip): one workgroup per block of query rows streams the
//      key/value tiles and sums its rows' dQ itself, with no atomics.
// dq, dk and dv are all bitwise deterministic.
#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kBwdKeys = 128;             // keys per workgroup
constexpr int kBwdRows = 64;              // query rows per tile

// The dK/dV grid walks key/value heads in chunks of this many (one per XCD).
constexpr int kBwdHeadChunk = 8;
static_assert(kBwdHeadChunk == 8, "the grid order maps head chunks onto the 8 XCDs");

// Q and dO tiles (kBwdRows rows) arrive by direct-to-LDS loads into a
// ring, unpadded, with the 16-byte chunks of each row XOR-swizzled
// so that both the 128-bit row reads (16 rows, one chunk column) and the
// transposed reads (4 rows x 64 bytes) are free of bank conflicts.
template <int D> struct BwdCfg {
  static constexpr int ROWB = 2 * D;                      // Q/dO tile row bytes
  static constexpr int TILEB = kBwdRows * ROWB;           // one Q (or dO) tile
  static constexpr int CPR = D / 8;                       // 16-byte chunks per row
  static constexpr int RPW = 1024 / ROWB;                 // rows per wave-wide 1 KB load
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
//
// Each 32-key group of the workgroup's 128 keys is split over two waves that
// share a SIMD (waves w and w + 4 of the 8): the "S" wave holds the keys' K rows,
// forms S = Q K^T and P for query tile s, accumulates dV^T += dO^T P and
// passes P (bf16) through LDS; the "dP" wave holds the (negated) V rows and,
// one tile behind, forms dP = dO V^T for tile s - 1, dS = P (dP - D) from
// the P its partner wrote in the previous step, and accumulates
// dK^T += Q^T dS. Each wave does two of the four products in ≈200
// registers, so two waves fit on a SIMD: while one waits for LDS or its
// vector work, the other feeds the matrix core, and each wave reads half
// the LDS bytes per tile. (One wave per SIMD doing all four products in 376
// registers was LDS-issue bound at 0.50 MFMA busy; this split is 2.6-3.7 %
// faster over the whole backward. dS uses P rounded to bf16, as passed.)
// The query tiles (and, with shared key/value heads, the tiles of every
// head of the group in turn) form one stream; step s loads tile s + 1 into
// a 3-slot ring, the S waves run tile s and the dP waves tile s - 1 (the
// slot loaded in step s is the one tile s - 2 used), so there are n + 1
// steps, each closed by the workgroup barrier that publishes the next tile
// and the P just written.
constexpr int kPairWaves = 8;
constexpr int kPairSlots = 3;

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(64 * kPairWaves, 1)
bwd_dkdv_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                const float* __restrict__ L2vec, const float* __restrict__ Dvec,
                uint16_t* __restrict__ dK, uint16_t* __restrict__ dV,
                int N, int n_kblocks, int n_kvheads, int group, float c2, float scale) {
  using C = BwdCfg<D>;
  constexpr int NDMA = C::TILEB / 1024 / kPairWaves;  // wave-wide loads per wave and tensor
  static_assert(C::TILEB % (1024 * kPairWaves) == 0, "tile must split into whole wave-wide loads");
  // ring slot s: Q tile at qd + (2s) TILEB, dO tile at qd + (2s+1) TILEB
  __shared__ __attribute__((aligned(1024))) char qd[2 * kPairSlots * C::TILEB];
  __shared__ __attribute__((aligned(16))) float rowstat[kPairSlots][2][kBwdRows];  // [slot][lse, D][row]
  // P of the S waves, double-buffered: [buffer][key group][query block][16-row half][lane], 16 B each
  __shared__ __attribute__((aligned(16))) char pbuf[2 * 4 * 2 * 2 * 64 * 16];
  FA_LDS char* qdl = (FA_LDS char*)qd;
  FA_LDS char* pbl = (FA_LDS char*)pbuf;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool s_wave = w < 4;  // S, P, dV; else dP, dS, dK (uniform per wave)
  const int kg = w & 3;       // key group of 32 (shared by waves w and w + 4, one SIMD)
  const int h = lane >> 5, n = lane & 31;
  // workgroup -> (key/value head, key block). The grid takes the heads in
  // chunks of kBwdHeadChunk and, inside a chunk, goes key-block-major:
  // workgroup b runs on XCD b % 8, so each XCD keeps to one head of the chunk
  // and its concurrent key blocks share that head's query tiles in L2, and
  // under a causal mask the longest key blocks (the first ones) start first.
  // Small causal launches (each XCD holding 4 or 8 heads and at most 256
  // workgroups, 8 per compute unit) take each XCD's heads 4 at a time with
  // their key blocks longest first across the 4, so the blocks that start
  // last are short ones (the causal B4 H16 N4096 backward: 2.4 % faster,
  // bitwise the same); with more work per unit the tail weighs little and
  // one head per XCD keeps its query tiles in L2.
  int kbi, kvbh;
  if (CAUSAL && n_kvheads % (4 * kBwdHeadChunk) == 0 && n_kvheads <= 8 * kBwdHeadChunk &&
      n_kvheads / kBwdHeadChunk * n_kblocks <= 256) {
    const int x = blockIdx.x & 7, jx = blockIdx.x >> 3;
    const int g = jx / (4 * n_kblocks), rr = jx - g * 4 * n_kblocks;
    kbi = __builtin_amdgcn_readfirstlane(rr >> 2);
    kvbh = __builtin_amdgcn_readfirstlane((4 * g + (rr & 3)) * kBwdHeadChunk + x);
  } else {
    const int chunk = blockIdx.x / (kBwdHeadChunk * n_kblocks);
    const int r = blockIdx.x - chunk * (kBwdHeadChunk * n_kblocks);
    const int cc = min(kBwdHeadChunk, n_kvheads - kBwdHeadChunk * chunk);
    kbi = __builtin_amdgcn_readfirstlane(r / cc);
    kvbh = __builtin_amdgcn_readfirstlane(kBwdHeadChunk * chunk + r - kbi * cc);
  }
  const int kb0 = __builtin_amdgcn_readfirstlane(kbi * kBwdKeys);
  const int key = kb0 + 32 * kg + n;
  const size_t head = (size_t)kvbh * N * D;

  // this lane's key row as the MFMA B operand: K (S waves) or -V (dP waves:
  // V enters dP only; its products start from D and yield D - dP)
  bf16x8_t bfr[D / 16];
  {
    const uint16_t* src = (s_wave ? K : V) + head + (size_t)key * D + 8 * h;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      u32x4_t a = {0u, 0u, 0u, 0u};
      if (key < N) a = *(const u32x4_t*)(src + 16 * c);
      if (!s_wave) a ^= 0x80008000u;
      bfr[c] = __builtin_bit_cast(bf16x8_t, a);
    }
  }
#pragma unroll
  for (int c = 0; c < D / 16; ++c) asm volatile("" :: "v"(bfr[c]));
  __builtin_amdgcn_s_waitcnt(0);

  f32x16_t acc[D / 32];
#pragma unroll
  for (int j = 0; j < D / 32; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[j][i] = 0.f;

  // ---- tile loads: all 8 waves share them (wave w fills 1 KB blocks w*NDMA ..)
  uint32_t qd_off[NDMA];
#pragma unroll
  for (int i = 0; i < NDMA; ++i) {
    const int rr = (w * NDMA + i) * C::RPW + lane / C::CPR;
    qd_off[i] = rr * C::ROWB + 16 * ((lane % C::CPR) ^ qswz<D>(rr));
  }
  // tile t of query head g of the group into ring slot `slot` (rows past N
  // read as zeros through the buffer resources' range, and are masked)
  auto load_item = [&](int g, int t, int slot) {
    const int bh = kvbh * group + g;
    const int q0 = t * kBwdRows;
    const uint32_t bytes = (uint32_t)min(N - q0, kBwdRows) * C::ROWB;
    const i32x4_t qr = buffer_rsrc(Q + ((size_t)bh * N + q0) * D, bytes);
    const i32x4_t gr = buffer_rsrc(dO + ((size_t)bh * N + q0) * D, bytes);
    FA_LDS char* dq_ = qdl + (2 * slot) * C::TILEB + w * NDMA * 1024;
    FA_LDS char* dg_ = qdl + (2 * slot + 1) * C::TILEB + w * NDMA * 1024;
    const int lim = N - 1 - q0;
#pragma unroll
    for (int i = 0; i < NDMA; ++i) {
      dma16_buf(qr, qd_off[i], dq_ + i * 1024);
      dma16_buf(gr, qd_off[i], dg_ + i * 1024);
    }
    if (w < 2) {  // wave 0: the rows' lse * log2(e), wave 1: their D
      const char* src = (const char*)((w == 0 ? L2vec : Dvec) + (size_t)bh * N + q0);
      dma4(src, 4u * (uint32_t)min(lane, lim), (FA_LDS char*)&rowstat[slot][w][0]);
    }
  };

  // LDS read offsets within a tile. Row reads (A operands of S and dP): row
  // n (+32 qb), logical chunk 2c + h, at row_off ^ (32 c). Transposed reads
  // (dO^T, Q^T): rows 4h + q (+16 jj, +32 qb) and 8 more, columns
  // 32 j + 16 x + 4 (lane & 3), at tr_off ^ (64 j).
  const int row_off = n * C::ROWB + 16 * (h ^ qswz<D>(n));
  const int tr_row = 4 * h + ((lane >> 2) & 3);
  const int tr_chunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int tr_off0 = tr_row * C::ROWB + 16 * (tr_chunk ^ qswz<D>(tr_row)) + 8 * (lane & 1);
  const int tr_off1 = (tr_row + 8) * C::ROWB + 16 * (tr_chunk ^ qswz<D>(tr_row + 8)) + 8 * (lane & 1);
  // this lane's 16-byte slot of P (query block qb, half jj) in buffer b
  auto p_slot = [&](int b, int qb, int jj) {
    return pbl + ((((b * 4 + kg) * 2 + qb) * 2 + jj) * 64 + lane) * 16;
  };

  const int n_qtiles = (N + kBwdRows - 1) / kBwdRows;
  const int t_first = CAUSAL ? kb0 / kBwdRows : 0;
  const int n_per = n_qtiles - t_first;
  const int n_items = __builtin_amdgcn_readfirstlane(group * n_per);
  const bool keys_tail = kb0 + kBwdKeys > N;
  // tiles with invisible pairs: the causal diagonal (below t_inner) and a
  // ragged last tile (from t_tail); a key block reaching past N masks all
  const int t_inner = keys_tail ? n_qtiles
                                : min(n_qtiles, CAUSAL ? (kb0 + kBwdKeys - 1) / kBwdRows + 1 : 0);
  const int t_tail = keys_tail ? 0 : (N / kBwdRows);

  constexpr int NC = D / 16;        // S/dP slices per query block
  constexpr int NB = 2 * (D / 32);  // dV/dK slices per query block (jj, j)
  auto rread = [&](const FA_LDS char* base, int ro, int qb, int c) {
    return *(const FA_LDS bf16x8_t*)(base + qb * 32 * C::ROWB + (ro ^ (32 * c)));
  };
  auto tread = [&](const FA_LDS char* base, int to0, int to1, int qb, int m) {
    const int jj = m / (D / 32), j = m % (D / 32);
    const int rb = (qb * 32 + 16 * jj) * C::ROWB;
    return concat8(lds_read_tr4(base + rb + (to0 ^ (64 * j))), lds_read_tr4(base + rb + (to1 ^ (64 * j))));
  };

  // ---- S wave: S, P (stored for the partner), dV for the tile in slot sl
  // (masked: the tile has invisible pairs; a uniform branch around the mask)
  auto item_s = [&](int q0, int sl, int pb_w, bool masked) __attribute__((always_inline)) {
    const FA_LDS char* Qs = qdl + (2 * sl) * C::TILEB;
    const FA_LDS char* Gs = qdl + (2 * sl + 1) * C::TILEB;
    int ro = row_off, to0 = tr_off0, to1 = tr_off1;
    asm volatile("" : "+v"(ro), "+v"(to0), "+v"(to1));
    f32x4_t st[2][4];  // the rows' lse * log2(e), lane's rows 8g + 4h .. + 3
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int g = 0; g < 4; ++g) st[qb][g] = *(const FA_LDS f32x4_t*)&rowstat[sl][0][qb * 32 + 8 * g + 4 * h];
    f32x16_t sc[2];
    bf16x8_t pb[2][2];
    auto mask = [&](int qb) {
      const int qlo = (CAUSAL ? key : 0) - q0 - qb * 32 - 4 * h;
      const int qhi = (key < N ? N : 0) - q0 - qb * 32 - 4 * h;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int qo = 8 * (i >> 2) + (i & 3);
        if (qo < qlo || qo >= qhi) sc[qb][i] = -INFINITY;
      }
    };
    auto p_pair = [&](int qb, int pr) {
      const int i = 2 * pr, g = i >> 2, e = i & 3;
      const float p0 = exp2_fast(fmaf(sc[qb][i], c2, -st[qb][g][e]));
      const float p1 = exp2_fast(fmaf(sc[qb][i + 1], c2, -st[qb][g][e + 1]));
      const bf16x2_t pp = to_bf16x2(p0, p1);
      pb[qb][i >> 3][i & 7] = pp[0];
      pb[qb][i >> 3][(i & 7) + 1] = pp[1];
    };
    bf16x8_t ra[NC], ta[NB];
    ra[0] = rread(Qs, ro, 0, 0);
    ra[1] = rread(Qs, ro, 0, 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < NC; ++c) {  // S of block 0
      const int cn = c + 2;
      if (cn < NC) ra[cn] = rread(Qs, ro, 0, cn);
      else ra[cn - NC] = rread(Qs, ro, 1, cn - NC);
      const f32x16_t z = {};
      sc[0] = mfma_32x32x16(ra[c], bfr[c], c == 0 ? z : sc[0]);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (masked) mask(0);
#pragma unroll
    for (int c = 0; c < NC; ++c) {  // S of block 1, P of block 0
      const int cn = c + 2;
      if (cn < NC) ra[cn] = rread(Qs, ro, 1, cn);
      else ta[cn - NC] = tread(Gs, to0, to1, 0, cn - NC);
      const f32x16_t z = {};
      sc[1] = mfma_32x32x16(ra[c], bfr[c], c == 0 ? z : sc[1]);
#pragma unroll
      for (int pr = c * 8 / NC; pr < (c + 1) * 8 / NC; ++pr) p_pair(0, pr);
      __builtin_amdgcn_sched_barrier(0);
    }
    *(FA_LDS bf16x8_t*)p_slot(pb_w, 0, 0) = pb[0][0];
    *(FA_LDS bf16x8_t*)p_slot(pb_w, 0, 1) = pb[0][1];
    if (masked) mask(1);
#pragma unroll
    for (int m = 0; m < NB; ++m) {  // dV over block 0, P of block 1
      const int mn = m + 2;
      if (mn < NB) ta[mn] = tread(Gs, to0, to1, 0, mn);
      else ta[mn - NB] = tread(Gs, to0, to1, 1, mn - NB);
      const int jj = m / (D / 32), j = m % (D / 32);
#pragma unroll
      for (int pr = m * 8 / NB; pr < (m + 1) * 8 / NB; ++pr) p_pair(1, pr);
      acc[j] = mfma_32x32x16(ta[m], pb[0][jj], acc[j]);
      __builtin_amdgcn_sched_barrier(0);
    }
    *(FA_LDS bf16x8_t*)p_slot(pb_w, 1, 0) = pb[1][0];
    *(FA_LDS bf16x8_t*)p_slot(pb_w, 1, 1) = pb[1][1];
#pragma unroll
    for (int m = 0; m < NB; ++m) {  // dV over block 1
      const int mn = m + 2;
      if (mn < NB) ta[mn] = tread(Gs, to0, to1, 1, mn);
      const int jj = m / (D / 32), j = m % (D / 32);
      acc[j] = mfma_32x32x16(ta[m], pb[1][jj], acc[j]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- dP wave: dP, dS (with its partner's P), dK for the tile in slot sl
  auto item_dp = [&](int sl, int pb_r) __attribute__((always_inline)) {
    const FA_LDS char* Qs = qdl + (2 * sl) * C::TILEB;
    const FA_LDS char* Gs = qdl + (2 * sl + 1) * C::TILEB;
    int ro = row_off, to0 = tr_off0, to1 = tr_off1;
    asm volatile("" : "+v"(ro), "+v"(to0), "+v"(to1));
    f32x4_t st[2][4];  // the rows' D
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int g = 0; g < 4; ++g) st[qb][g] = *(const FA_LDS f32x4_t*)&rowstat[sl][1][qb * 32 + 8 * g + 4 * h];
    bf16x8_t pin[2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) pin[qb][jj] = *(const FA_LDS bf16x8_t*)p_slot(pb_r, qb, jj);
    f32x16_t dp[2];
    bf16x8_t dsb[2][2];
    auto dinit = [&](int qb) {
      f32x16_t v;
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = st[qb][i >> 2][i & 3];
      return v;
    };
    // dp holds D - dP: dS = P (dP - D) = -P (D - dP)
    auto ds_pair = [&](int qb, int pr) {
      const int i = 2 * pr;
      const float p0 = (float)pin[qb][i >> 3][i & 7];
      const float p1 = (float)pin[qb][i >> 3][(i & 7) + 1];
      const bf16x2_t dd = to_bf16x2(p0 * -dp[qb][i], p1 * -dp[qb][i + 1]);
      dsb[qb][i >> 3][i & 7] = dd[0];
      dsb[qb][i >> 3][(i & 7) + 1] = dd[1];
    };
    bf16x8_t rg[NC], ta[NB];
    rg[0] = rread(Gs, ro, 0, 0);
    rg[1] = rread(Gs, ro, 0, 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < NC; ++c) {  // dP of block 0
      const int cn = c + 2;
      if (cn < NC) rg[cn] = rread(Gs, ro, 0, cn);
      else rg[cn - NC] = rread(Gs, ro, 1, cn - NC);
      dp[0] = mfma_32x32x16(rg[c], bfr[c], c == 0 ? dinit(0) : dp[0]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // (issue priority while this wave's dS work is interleaved with its
    // products, so its MFMAs win the matrix core from the S wave's: 0.4 %)
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int c = 0; c < NC; ++c) {  // dP of block 1, dS of block 0
      const int cn = c + 2;
      if (cn < NC) rg[cn] = rread(Gs, ro, 1, cn);
      else ta[cn - NC] = tread(Qs, to0, to1, 0, cn - NC);
      dp[1] = mfma_32x32x16(rg[c], bfr[c], c == 0 ? dinit(1) : dp[1]);
#pragma unroll
      for (int pr = c * 8 / NC; pr < (c + 1) * 8 / NC; ++pr) ds_pair(0, pr);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int m = 0; m < NB; ++m) {  // dK over block 0, dS of block 1
      const int mn = m + 2;
      if (mn < NB) ta[mn] = tread(Qs, to0, to1, 0, mn);
      else ta[mn - NB] = tread(Qs, to0, to1, 1, mn - NB);
      const int jj = m / (D / 32), j = m % (D / 32);
#pragma unroll
      for (int pr = m * 8 / NB; pr < (m + 1) * 8 / NB; ++pr) ds_pair(1, pr);
      acc[j] = mfma_32x32x16(ta[m], dsb[0][jj], acc[j]);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int m = 0; m < NB; ++m) {  // dK over block 1
      const int mn = m + 2;
      if (mn < NB) ta[mn] = tread(Qs, to0, to1, 1, mn);
      const int jj = m / (D / 32), j = m % (D / 32);
      acc[j] = mfma_32x32x16(ta[m], dsb[1][jj], acc[j]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- the stream: step s loads item s + 1, the S waves run item s and the
  // dP waves item s - 1; (g_ld, t_ld) is the item being loaded, t_s the S
  // waves' tile
  // (each role runs its own copy of the loop, with the same loads and
  // barriers, so the compiler keeps each role's registers where they are)
  int g_ld = 0, t_ld = t_first;
  load_item(g_ld, t_ld, 0);
  wait_loads_and_barrier<0>();
  int t_s = t_ld;
  auto advance = [&]() {
    if (++t_ld == n_qtiles) { t_ld = t_first; ++g_ld; }
  };
  advance();
  if (s_wave) {
    for (int st_i = 0; st_i <= n_items; ++st_i) {
      if (st_i + 1 < n_items) load_item(g_ld, t_ld, (st_i + 1) % kPairSlots);
      if (st_i < n_items) item_s(t_s * kBwdRows, st_i % kPairSlots, st_i & 1, t_s < t_inner || t_s >= t_tail);
      // the next item's tile, row statistics and this step's P are in LDS
      wait_loads_and_barrier<0>();
      t_s = t_ld;
      advance();
    }
  } else {
    for (int st_i = 0; st_i <= n_items; ++st_i) {
      if (st_i + 1 < n_items) load_item(g_ld, t_ld, (st_i + 1) % kPairSlots);
      if (st_i >= 1) item_dp((st_i - 1) % kPairSlots, (st_i - 1) & 1);
      wait_loads_and_barrier<0>();
      advance();
    }
  }

  // dV = (dV^T)^T from the S waves, dK = scale (dK^T)^T from the dP waves
  if (key < N) {
    uint16_t* dst = (s_wave ? dV : dK) + head + (size_t)key * D;
    const float f = s_wave ? 1.f : scale;
#pragma unroll
    for (int j = 0; j < D / 32; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const bf16x2_t a01 = to_bf16x2(f * acc[j][4 * g], f * acc[j][4 * g + 1]);
        const bf16x2_t a23 = to_bf16x2(f * acc[j][4 * g + 2], f * acc[j][4 * g + 3]);
        const u32x2_t vv = {__builtin_bit_cast(uint32_t, a01), __builtin_bit_cast(uint32_t, a23)};
        *(u32x2_t*)(dst + 32 * j + 8 * g + 4 * h) = vv;
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
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3((unsigned)blocks), dim3(64 * kPairWaves), 0,
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
