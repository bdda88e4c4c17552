// dQ of exact attention with recomputation, bf16 in/out, fp32 accumulation, gfx950.
//
// "Attention and KV Compression", section "Recomputation in the backward
// pass": the probabilities are not stored; every tile recomputes them from
// Q, K and the saved per-row logsumexp. For the query gradient,
//     dQ = scale * dS K,   dS = P * (dP - D),   dP = dO V^T,   P = exp(S - lse),
// with D = rowsum(dO * O) from the preprocess kernel (the derivative of the
// score / softmax / weight definition; the pages give no formula).
//
// Structure (the forward's, with the softmax replaced by the gradient step):
//   * A workgroup owns 32*NW query rows; wave w owns 32 of them. Its Q and dO
//     rows stay in registers as the B operands of S^T = K Q^T and
//     dP^T = V dO^T (v_mfma_f32_32x32x16_bf16), so each lane owns ONE query
//     row: lse and D are per-lane scalars, and no cross-lane reduction is
//     needed anywhere.
//   * K and V tiles (BN keys) stream through a ring of S LDS slots filled by
//     direct-to-LDS loads, several tiles ahead, one barrier per tile.
//   * dQ^T += K^T dS^T on the matrix cores: dS^T (bf16) comes straight from
//     the registers that hold dP^T and P^T, and K^T is read from K's
//     row-major LDS tile with ds_read_b64_tr_b16 (K is therefore read both by
//     rows and transposed, and its 16-byte chunks are swizzled for both).
//   * A step is straight-line code in scheduling slices, one or two MFMAs
//     each: the scores and dP of the tile's second 32-key block run on the
//     matrix cores while the vector unit computes the first block's P and
//     dS, and the second block's P and dS overlap the first dQ products.
//     LDS operands are read two slices ahead; every accumulator sums in the
//     order of the plain loop nest, so the schedule does not change results.
//   * No atomics: every query row's gradient is summed by one wave, so dq is
//     deterministic; the price is recomputing S and dP a second time (the
//     dK/dV kernel computes them too).
//   * Causal: a query block's key range ends at its last row; only tiles on
//     the diagonal or the ragged tail are masked (tail rows are loaded from
//     key N-1, finite, and masked).
#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

template <int D, int NW, int BN, int S>
struct DqCfg {
  static constexpr int BM = 32 * NW;              // query rows per workgroup
  static constexpr int NT = 64 * NW;              // threads
  static constexpr int ROWB = 2 * D;              // bytes per K/V row in LDS
  static constexpr int TILEB = BN * ROWB;         // one K (or V) tile
  static constexpr int CPR = D / 8;               // 16-byte chunks per row
  static constexpr int RPW = 1024 / ROWB;         // rows per wave-wide 1 KB load
  static constexpr int NDMA = TILEB / 1024 / NW;  // wave-wide loads per wave, tile and tensor
  static constexpr int LDS_BYTES = 2 * S * TILEB; // K slots then V slots
  // DMAs a wave may leave in flight at the end of a step: those of the
  // tiles issued after the one the next step reads
  static constexpr int INFLIGHT = 2 * (S - 2) * NDMA;
  static_assert(TILEB % (1024 * NW) == 0, "a tile must split into whole wave-wide loads");
  static_assert(S >= 2 && (S & (S - 1)) == 0 && INFLIGHT <= 63, "stages");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS capacity");
  static_assert(BN % 32 == 0 && (D == 64 || D == 128), "tile shape");
};

// Swizzle of K tiles (row reads of 16 rows and transposed reads of 4 rows x
// 64 bytes both conflict-free): bits 3..2 from the row's position within a
// group of 4, bits 1..0 from the next row bits (per 256-byte bank line).
template <int D>
__device__ __forceinline__ int kdual_swz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}
// Swizzle of V tiles (row reads only): 16 consecutive rows, 16 slots.
template <int D>
__device__ __forceinline__ int vrow_swz(int r) {
  constexpr int RPL = 128 / D;
  return (r / RPL) & (D / 8 - 1);
}

template <int D, int NW, int BN, int S, bool CAUSAL>
__global__ void __launch_bounds__(64 * NW)
bwd_dq_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
              const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
              const float* __restrict__ LSE, const float* __restrict__ Dvec,
              uint16_t* __restrict__ dQ, int N, int n_qtiles, int group, float c2, float scale) {
  using C = DqCfg<D, NW, BN, S>;
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];
  FA_LDS char* lds = (FA_LDS char*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;  // which 16 of each 32 keys this lane holds
  const int n = lane & 31;  // this lane's query row within the wave

  // ---- workgroup -> (head, query block): XCD-aware, longest causal first
  const int G = gridDim.x, b = blockIdx.x;
  const int xcd = b & 7, jx = b >> 3, per = G >> 3, rem = G & 7;
  const int logical = xcd * per + min(xcd, rem) + jx;
  int bh, t;
  // Causal, when each XCD's share is 4 or 8 whole heads: a group of 4 heads
  // has its blocks go longest first across the 4, so the blocks that start
  // last on an XCD are short ones. (With more heads per XCD the tail is a
  // small part of the time and one head in flight per XCD keeps its L2 hits.)
  if (CAUSAL && rem == 0 && per % (4 * n_qtiles) == 0 && per <= 8 * n_qtiles) {
    const int gi = __builtin_amdgcn_readfirstlane(logical / (4 * n_qtiles));
    const int r = logical - gi * 4 * n_qtiles;
    bh = gi * 4 + (r & 3);
    t = n_qtiles - 1 - (r >> 2);
  } else {
    bh = __builtin_amdgcn_readfirstlane(logical / n_qtiles);
    t = logical - bh * n_qtiles;
    if (CAUSAL) t = n_qtiles - 1 - t;
  }
  const int q0 = __builtin_amdgcn_readfirstlane(t * C::BM);
  const int row0 = __builtin_amdgcn_readfirstlane(q0 + 32 * w);
  const int qrow = row0 + n;
  const size_t head = (size_t)bh * N * D;
  // consecutive query heads share a key/value head: (b, h) reads (b, h / group)
  const size_t kvhead = (size_t)__builtin_amdgcn_readfirstlane(bh / group) * N * D;
  const uint16_t* Kh = K + kvhead;
  const uint16_t* Vh = V + kvhead;

  const int kv_end = CAUSAL ? min(N, q0 + C::BM) : N;
  const int n_tiles = __builtin_amdgcn_readfirstlane((kv_end + BN - 1) / BN);

  // ---- K/V tile loads (as in the forward): lane `lane` of wave-wide load i
  // fills the 16-byte LDS slot `lane` of 1 KB block w*NDMA + i
  uint32_t dk_off[C::NDMA], dv_off[C::NDMA];
#pragma unroll
  for (int i = 0; i < C::NDMA; ++i) {
    const int r = (w * C::NDMA + i) * C::RPW + lane / C::CPR;
    const int phys = lane % C::CPR;
    dk_off[i] = r * C::ROWB + 16 * (phys ^ kdual_swz<D>(r));
    dv_off[i] = r * C::ROWB + 16 * (phys ^ vrow_swz<D>(r));
  }
  // tile t goes to ring slot t % S; past the last tile the last one repeats
  // into the (unused) slot, so every step issues the same number of loads
  auto load_tile = [&](const uint16_t* src, int tt, int slot0, const uint32_t (&off)[C::NDMA]) {
    const int slot = slot0 + (tt & (S - 1));
    const int k0 = min(tt, n_tiles - 1) * BN;
    const char* base = (const char*)(src + (size_t)k0 * D);
    FA_LDS char* dst = lds + slot * C::TILEB + w * C::NDMA * 1024;
    if (k0 + BN <= N) {
#pragma unroll
      for (int i = 0; i < C::NDMA; ++i) dma16(base, off[i], dst + i * 1024);
    } else {
      const int lim = N - 1 - k0;
#pragma unroll
      for (int i = 0; i < C::NDMA; ++i)
        dma16(base, (uint32_t)min((int)(off[i] / C::ROWB), lim) * C::ROWB + off[i] % C::ROWB,
              dst + i * 1024);
    }
  };

  // ---- this lane's query row: Q and dO as B operands, lse and D scalars
  bf16x8_t qf[D / 16], gf[D / 16];
  float lse2 = 0.f, Dl = 0.f;
  {
    const uint16_t* Qr = Q + head + (size_t)qrow * D;
    const uint16_t* Gr = dO + head + (size_t)qrow * D;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      u32x4_t x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
      if (qrow < N) {
        x = *(const u32x4_t*)(Qr + 16 * c + 8 * h);
        y = *(const u32x4_t*)(Gr + 16 * c + 8 * h);
      }
      qf[c] = __builtin_bit_cast(bf16x8_t, x);
      gf[c] = __builtin_bit_cast(bf16x8_t, y);
    }
    if (qrow < N) {
      lse2 = LSE[(size_t)bh * N + qrow] * kLog2e;
      Dl = Dvec[(size_t)bh * N + qrow];
    }
  }
  // take delivery of these loads before the tile loads start
#pragma unroll
  for (int c = 0; c < D / 16; ++c) asm volatile("" :: "v"(qf[c]), "v"(gf[c]));
  asm volatile("" :: "v"(lse2), "v"(Dl));

  // LDS read offsets within a tile (bytes). Row reads: row n (+32 kb),
  // logical chunk 2c + h at off ^ (32 c). Transposed K reads: rows 4h + q
  // (+16 multiples) and 8 more, columns 32 j + 16 x + 4 (lane & 3), at
  // tr_off[hi] ^ (64 j).
  const int krow_off = n * C::ROWB + 16 * (h ^ kdual_swz<D>(n));
  const int vrow_off = n * C::ROWB + 16 * (h ^ vrow_swz<D>(n));
  const int tr_row = 4 * h + ((lane >> 2) & 3);
  const int tr_chunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int tr_off0 = tr_row * C::ROWB + 16 * (tr_chunk ^ kdual_swz<D>(tr_row)) + 8 * (lane & 1);
  const int tr_off1 =
      (tr_row + 8) * C::ROWB + 16 * (tr_chunk ^ kdual_swz<D>(tr_row + 8)) + 8 * (lane & 1);

  f32x16_t acc[D / 32];  // dQ^T block: lane holds dQ[qrow][32j + 8(i/4) + 4h + i%4]
#pragma unroll
  for (int j = 0; j < D / 32; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[j][i] = 0.f;

  // ---- pipeline: step u reads K(u), V(u) and issues tile u+S-1, which
  // replaces tile u-1 (last read in step u-1, before its closing barrier).
  // At the end of step u the next step needs tile u+1, after which tiles
  // u+2 .. u+S-1 were issued: INFLIGHT DMAs may stay outstanding.
#pragma unroll
  for (int tt = 0; tt + 1 < S; ++tt) {
    load_tile(Kh, tt, 0, dk_off);
    load_tile(Vh, tt, S, dv_off);
  }
  wait_loads_and_barrier<C::INFLIGHT>();

  // ---- one step (key tile u) as an explicit schedule of scheduling slices:
  //   S^T, dP^T of key block kb (32 keys; 2 MFMAs per d chunk), kb-major,
  //     with the gradient of block kb-1 on the vector unit;
  //   dQ^T += K^T dS^T, 16-key group major, with the last block's gradient
  //     in the first three quarters of its slices (each group's dS is
  //     complete before its first product).
  // Each accumulator sums in the same order as a plain loop nest would. The
  // LDS operands of a slice are read LA slices ahead (row reads of K and V
  // for S and dP, transposed reads of K for dQ). MASKED: the tile reaches
  // past this wave's rows (causal) or past N, and P is masked.
  constexpr int NCH = D / 16;        // d chunks: S/dP slices per key block
  constexpr int NKB = BN / 32;       // key blocks of 32
  constexpr int NA = NKB * NCH;      // S/dP slices
  constexpr int NJ = D / 32;         // dQ^T row blocks
  constexpr int NQ = (BN / 16) * NJ; // dQ slices
  constexpr int LA = 2;
  constexpr int PPS_A = 8 / NCH;     // gradient pairs per S/dP slice (8 pairs per key block)
  constexpr int NQG = 3 * NJ;        // dQ slices that carry the last block's gradient
  static_assert(8 % NCH == 0 && NKB == 2, "slicing: two 32-key blocks per tile");
  const int u_full = __builtin_amdgcn_readfirstlane(
      CAUSAL ? min((row0 + 1) / BN, N / BN) : N / BN);  // tiles before it need no mask
  auto step = [&](int u, auto masked) {
    constexpr bool MASKED = decltype(masked)::value;
    load_tile(Kh, u + S - 1, 0, dk_off);
    load_tile(Vh, u + S - 1, S, dv_off);
    const int slot = u & (S - 1);
    // per-step LDS addresses through an empty asm statement so the per-chunk
    // XORs are formed here rather than kept live across the loop
    int ka = (int)(uintptr_t)(lds + slot * C::TILEB) + krow_off;
    int va = (int)(uintptr_t)(lds + (S + slot) * C::TILEB) + vrow_off;
    int t0 = (int)(uintptr_t)(lds + slot * C::TILEB) + tr_off0;
    int t1 = (int)(uintptr_t)(lds + slot * C::TILEB) + tr_off1;
    asm volatile("" : "+v"(ka), "+v"(va), "+v"(t0), "+v"(t1));
    const int lim = (CAUSAL ? min(qrow, N - 1) : N - 1) - u * BN - 4 * h;

    bf16x8_t rk[NA], rv[NA], rt[NQ];
    auto issue = [&](int x) {
      if (x < NA) {
        const int kb = x / NCH, c = x % NCH;
        rk[x] = *(const FA_LDS bf16x8_t*)((FA_LDS char*)(uintptr_t)(ka ^ (32 * c)) + kb * 32 * C::ROWB);
        rv[x] = *(const FA_LDS bf16x8_t*)((FA_LDS char*)(uintptr_t)(va ^ (32 * c)) + kb * 32 * C::ROWB);
      } else if (x < NA + NQ) {
        const int y = x - NA, kc = y / NJ, j = y % NJ;
        const int rb = ((kc >> 1) * 32 + 16 * (kc & 1)) * C::ROWB;
        rt[y] = concat8(lds_read_tr4((FA_LDS char*)(uintptr_t)(t0 ^ (64 * j)) + rb),
                        lds_read_tr4((FA_LDS char*)(uintptr_t)(t1 ^ (64 * j)) + rb));
      }
    };
    // P^T = exp(S^T - lse), dS^T = P^T (dP^T - D) -> bf16 for elements 2pr,
    // 2pr+1 of key block kb (lane holds keys 32kb + 8(i/4) + 4h + i%4)
    f32x16_t s[NKB], dp[NKB];
    bf16x8_t ds[BN / 16];
    auto grad_pair = [&](int kb, int pr) {
      const int i = 2 * pr;
      float p0 = exp2_fast(fmaf(s[kb][i], c2, -lse2));
      float p1 = exp2_fast(fmaf(s[kb][i + 1], c2, -lse2));
      if constexpr (MASKED) {
        if (kb * 32 + 8 * (i >> 2) + (i & 3) > lim) p0 = 0.f;
        if (kb * 32 + 8 * ((i + 1) >> 2) + ((i + 1) & 3) > lim) p1 = 0.f;
      }
      const bf16x2_t d2 = to_bf16x2(p0 * (dp[kb][i] - Dl), p1 * (dp[kb][i + 1] - Dl));
      ds[2 * kb + (i >> 3)][i & 7] = d2[0];
      ds[2 * kb + (i >> 3)][(i & 7) + 1] = d2[1];
    };

#pragma unroll
    for (int x = 0; x < LA; ++x) issue(x);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int x = 0; x < NA; ++x) {
      issue(x + LA);
      const int kb = x / NCH, c = x % NCH;
      const f32x16_t z = {};
      s[kb] = mfma_32x32x16(rk[x], qf[c], c == 0 ? z : s[kb]);
      dp[kb] = mfma_32x32x16(rv[x], gf[c], c == 0 ? z : dp[kb]);
      if (kb >= 1) {
#pragma unroll
        for (int pr = c * PPS_A; pr < (c + 1) * PPS_A; ++pr) grad_pair(kb - 1, pr);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int y = 0; y < NQ; ++y) {
      issue(NA + y + LA);
      const int kc = y / NJ, j = y % NJ;
      // its first half (pairs 0-3) is multiplied from slice 2 NJ on, its
      // second half from slice 3 NJ: spread over the first 3 NJ slices
      if (y < NQG) {
#pragma unroll
        for (int pr = y * 8 / NQG; pr < (y + 1) * 8 / NQG; ++pr) grad_pair(NKB - 1, pr);
      }
      acc[j] = mfma_32x32x16(rt[y], ds[kc], acc[j]);
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_loads_and_barrier<C::INFLIGHT>();
  };
  int u = 0;
  for (; u < min(u_full, n_tiles); ++u) step(u, std::false_type{});
  for (; u < n_tiles; ++u) step(u, std::true_type{});
  // no load may still be writing this workgroup's LDS when it exits
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- dq = scale * dQ, bf16
  if (qrow < N) {
    uint16_t* Dr = dQ + head + (size_t)qrow * D;
#pragma unroll
    for (int j = 0; j < D / 32; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const bf16x2_t a = to_bf16x2(scale * acc[j][4 * g], scale * acc[j][4 * g + 1]);
        const bf16x2_t bb = to_bf16x2(scale * acc[j][4 * g + 2], scale * acc[j][4 * g + 3]);
        u32x2_t packed = {__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, bb)};
        *(u32x2_t*)(Dr + 32 * j + 8 * g + 4 * h) = packed;
      }
  }
}

template <int D, int NW, int BN, int S, bool CAUSAL>
hipError_t launch(const void* q, const void* k, const void* v, const void* dO, const float* lse,
                  const float* Dvec, void* dq, const Problem& p, hipStream_t stream) {
  using C = DqCfg<D, NW, BN, S>;
  const int n_qtiles = (p.N + C::BM - 1) / C::BM;
  const long long grid = (long long)p.B * p.H * n_qtiles;
  hipLaunchKernelGGL((bwd_dq_kernel<D, NW, BN, S, CAUSAL>), dim3((unsigned)grid), dim3(C::NT), 0,
                     stream, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                     (const uint16_t*)dO, lse, Dvec, (uint16_t*)dq, p.N, n_qtiles, p.group(),
                     p.scale * kLog2e, p.scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_dq(const void* q, const void* k, const void* v, const void* dO,
                         const float* lse, const float* Dvec, void* dq, const Problem& p,
                         hipStream_t stream) {
  static_assert(DqCfg<128, 8, 64, 4>::BM == kFwdRowsPerBlock, "grid-size limit assumes 256-row blocks");
  if (p.d == 128)
    return p.causal ? launch<128, 8, 64, 4, true>(q, k, v, dO, lse, Dvec, dq, p, stream)
                    : launch<128, 8, 64, 4, false>(q, k, v, dO, lse, Dvec, dq, p, stream);
  return p.causal ? launch<64, 8, 64, 4, true>(q, k, v, dO, lse, Dvec, dq, p, stream)
                  : launch<64, 8, 64, 4, false>(q, k, v, dO, lse, Dvec, dq, p, stream);
}

}  // namespace fa
