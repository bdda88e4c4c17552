// Exact tiled attention forward, bf16 in / bf16 O + fp32 lse out, for gfx950.
//
// The method ("Attention and KV Compression", section "Tiling and online
// softmax"; "FlashAttention — how 100K-token attention fits in memory",
// sections "FlashAttention idea", "But softmax needs the whole row — right?",
// "Online softmax intuition"): a workgroup owns a block of query rows and
// streams blocks of keys and values past it. Each tile's scores exist only in
// registers; a running row maximum m, running denominator l and an fp32
// output accumulator are rescaled by 2^(m_old - m_new) when a tile raises the
// maximum; only O and the per-row logsumexp reach HBM.
//
// Mapping onto CDNA4:
//   * A workgroup has NW waves; wave w owns 32 query rows, held in registers
//     as the B operand of v_mfma_f32_32x32x16_bf16 (Q^T, d split in 16s).
//   * Scores are computed transposed, S^T = K Q^T (A = a K row-block read from
//     LDS with 128-bit reads), so each lane owns ONE query row and 16 of every
//     32 keys; the other 16 sit in lane l ^ 32. Row max / row sum are in-lane
//     plus one v_permlane32_swap.
//   * The output is accumulated transposed too, O^T += V^T P^T: P^T comes
//     straight from the score registers (rounded to bf16), and the V^T
//     operand is read from V's natural row-major LDS tile with
//     ds_read_b64_tr_b16. The contraction index order inside each 16-key MFMA
//     step follows the score registers' key order, which the two transposed
//     reads reproduce (rows 4h..4h+3 and 8+4h..8+4h+3 of each 16-key group).
//   * K and V tiles (BN keys) are double-buffered in LDS; the next tile's
//     global loads are issued before the current tile's math, and stored to
//     the other buffer after it, so one barrier per tile suffices.
//   * Causal: the key range of a query block ends at its last row; tiles
//     wholly after a wave's last row are skipped by that wave; only tiles
//     touching the diagonal or the ragged tail (keys >= N) are masked.
//   * Grid order: workgroups are dispatched round-robin over the 8 XCDs; the
//     block index is remapped so each XCD works through whole heads (K/V of a
//     head stay in that XCD's L2), longest causal query blocks first.
// Scores are kept in log2 units: s2 = s * scale * log2(e), so exp is v_exp_f32.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

template <int D, int NW, int BN>
struct FwdCfg {
  static constexpr int BM = 32 * NW;        // query rows per workgroup
  static constexpr int NT = 64 * NW;        // threads
  static constexpr int KSTRIDE = D + 8;     // bf16 per K row in LDS (16 B pad: conflict-free 128-bit row reads)
  static constexpr int VSTRIDE = D + 32;    // bf16 per V row in LDS (row pitch = 16 banks mod 64: conflict-free transposed reads)
  static constexpr int KTILE = BN * KSTRIDE;
  static constexpr int VTILE = BN * VSTRIDE;
  static constexpr int BUF = KTILE + VTILE; // one K+V buffer, in bf16 elements
  static constexpr int CHUNKS = BN * D / 8; // 16-byte chunks per K (or V) tile
  static constexpr int CPT = CHUNKS / NT;   // chunks per thread per tensor
  static constexpr int LDS_ELEMS = 2 * BUF;
  static_assert(CHUNKS % NT == 0, "tile must split evenly over threads");
  static_assert(BN % 32 == 0 && D % 32 == 0, "tile shape");
};

template <int D, int NW, int BN, bool CAUSAL>
__global__ void __launch_bounds__(64 * NW)
fwd_bf16_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                float* __restrict__ LSE, int N, int n_qtiles, float c2) {
  using C = FwdCfg<D, NW, BN>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[C::LDS_ELEMS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int h = lane >> 5;  // which 16 of each 32 keys this lane holds
  const int n = lane & 31;  // this lane's query row within the wave

  // ---- workgroup -> (head, query block): XCD-aware, longest causal first
  const int G = gridDim.x, b = blockIdx.x;
  const int xcd = b & 7, jx = b >> 3, per = G >> 3, rem = G & 7;
  const int logical = xcd * per + min(xcd, rem) + jx;
  const int bh = logical / n_qtiles;
  int t = logical - bh * n_qtiles;
  if (CAUSAL) t = n_qtiles - 1 - t;
  const int q0 = t * C::BM;
  const int row0 = q0 + 32 * w;
  const int qrow = row0 + n;
  const size_t head = (size_t)bh * N * D;
  const uint16_t* Qh = Q + head;
  const uint16_t* Kh = K + head;
  const uint16_t* Vh = V + head;

  // ---- Q^T operand: lane holds Q[qrow][16c + 8h .. +7]
  bf16x8_t qf[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    u32x4_t x = {0u, 0u, 0u, 0u};
    if (qrow < N) x = *(const u32x4_t*)(Qh + (size_t)qrow * D + 16 * c + 8 * h);
    qf[c] = __builtin_bit_cast(bf16x8_t, x);
  }

  const int kv_end = CAUSAL ? min(N, q0 + C::BM) : N;
  const int n_tiles = (kv_end + BN - 1) / BN;

  // ---- K/V tile staging: thread handles 16-byte chunks tid + i*NT
  u32x4_t kr[C::CPT], vr[C::CPT];
  auto gload = [&](int u) {
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int ch = tid + i * C::NT;
      const int r = ch / (D / 8), cc = ch % (D / 8);
      const int key = u * BN + r;
      u32x4_t zk = {0u, 0u, 0u, 0u}, zv = {0u, 0u, 0u, 0u};
      if (key < N) {
        zk = *(const u32x4_t*)(Kh + (size_t)key * D + cc * 8);
        zv = *(const u32x4_t*)(Vh + (size_t)key * D + cc * 8);
      }
      kr[i] = zk;
      vr[i] = zv;
    }
  };
  auto sstore = [&](int buf) {
    uint16_t* Ks = smem + buf * C::BUF;
    uint16_t* Vs = Ks + C::KTILE;
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int ch = tid + i * C::NT;
      const int r = ch / (D / 8), cc = ch % (D / 8);
      *(u32x4_t*)(Ks + r * C::KSTRIDE + cc * 8) = kr[i];
      *(u32x4_t*)(Vs + r * C::VSTRIDE + cc * 8) = vr[i];
    }
  };

  float m_run = -INFINITY;  // running max of s2 for row qrow
  float l_run = 0.f;        // running sum of 2^(s2 - m_run) over this lane's keys
  f32x16_t acc[D / 32];     // O^T block: lane holds O[qrow][32j + 8(i/4) + 4h + i%4]
#pragma unroll
  for (int j = 0; j < D / 32; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[j][i] = 0.f;

  gload(0);
  sstore(0);
  __syncthreads();

  for (int u = 0; u < n_tiles; ++u) {
    if (u + 1 < n_tiles) gload(u + 1);
    const int k0 = u * BN;
    const bool active = (row0 < N) && (!CAUSAL || k0 <= row0 + 31);
    if (active) {
      const uint16_t* Ks = smem + (u & 1) * C::BUF;
      const uint16_t* Vs = Ks + C::KTILE;

      // S^T = K Q^T for BN keys x 32 queries
      f32x16_t s[BN / 32];
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
#pragma unroll
        for (int c = 0; c < D / 16; ++c) {
          const bf16x8_t a = *(const bf16x8_t*)(Ks + (kb * 32 + n) * C::KSTRIDE + 16 * c + 8 * h);
          s[kb] = mfma_32x32x16(a, qf[c], s[kb]);
        }
      }

      // mask: only tiles that cross the diagonal or the ragged tail
      const bool need_mask = (CAUSAL && (k0 + BN - 1 > row0)) || (k0 + BN > N);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = k0 + kb * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
            if ((CAUSAL && key > qrow) || key >= N) s[kb][i] = -INFINITY;
          }
      }

      // online softmax update
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
      mx = halves_max(mx);
      const float m_new = fmaxf(m_run, mx * c2);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = exp2_fast(m_run - m_use);
      float lsum = 0.f;
      bf16x8_t p[BN / 16];
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const float p0 = exp2_fast(fmaf(s[kb][8 * jj + e], c2, -m_use));
            const float p1 = exp2_fast(fmaf(s[kb][8 * jj + e + 1], c2, -m_use));
            lsum += p0 + p1;
            const bf16x2_t pb = to_bf16x2(p0, p1);
            p[2 * kb + jj][e] = pb[0];
            p[2 * kb + jj][e + 1] = pb[1];
          }
      l_run = l_run * alpha + lsum;
      m_run = m_new;
#pragma unroll
      for (int j = 0; j < D / 32; ++j)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[j][i] *= alpha;

      // O^T += V^T P^T
      const int tr_row = 4 * h + ((lane >> 2) & 3);
      const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
      for (int kc = 0; kc < BN / 16; ++kc) {
        const int r = (kc >> 1) * 32 + 16 * (kc & 1) + tr_row;
#pragma unroll
        for (int j = 0; j < D / 32; ++j) {
          const uint16_t* vp = Vs + r * C::VSTRIDE + 32 * j + tr_col;
          const bf16x8_t a = concat8(lds_read_tr4(vp), lds_read_tr4(vp + 8 * C::VSTRIDE));
          acc[j] = mfma_32x32x16(a, p[kc], acc[j]);
        }
      }
    }
    if (u + 1 < n_tiles) sstore((u + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: O = acc / l, lse = ln(2) * (m + log2 l)
  if (qrow < N) {
    const float l_tot = halves_sum(l_run);
    const float inv = 1.f / l_tot;
    uint16_t* Orow = O + head + (size_t)qrow * D;
#pragma unroll
    for (int j = 0; j < D / 32; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const bf16x2_t a = to_bf16x2(acc[j][4 * g] * inv, acc[j][4 * g + 1] * inv);
        const bf16x2_t bb = to_bf16x2(acc[j][4 * g + 2] * inv, acc[j][4 * g + 3] * inv);
        u32x2_t packed = {__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, bb)};
        *(u32x2_t*)(Orow + 32 * j + 8 * g + 4 * h) = packed;
      }
    if (h == 0) LSE[(size_t)bh * N + qrow] = (m_run + log2_fast(l_tot)) * kLn2;
  }
}

template <int D, int NW, int BN, bool CAUSAL>
hipError_t launch(const void* q, const void* k, const void* v, void* o, float* lse,
                  const Problem& p, hipStream_t stream) {
  using C = FwdCfg<D, NW, BN>;
  const int n_qtiles = (p.N + C::BM - 1) / C::BM;
  const long long grid = (long long)p.B * p.H * n_qtiles;
  const float c2 = p.scale * kLog2e;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, BN, CAUSAL>), dim3((unsigned)grid), dim3(C::NT), 0, stream,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)o, lse,
                     p.N, n_qtiles, c2);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                           const Problem& p, hipStream_t stream) {
  static_assert(FwdCfg<128, 8, 64>::BM == kFwdRowsPerBlock, "grid-size limit assumes 256-row blocks");
  if (p.d == 128)
    return p.causal ? launch<128, 8, 64, true>(q, k, v, o, lse, p, stream)
                    : launch<128, 8, 64, false>(q, k, v, o, lse, p, stream);
  return p.causal ? launch<64, 8, 64, true>(q, k, v, o, lse, p, stream)
                  : launch<64, 8, 64, false>(q, k, v, o, lse, p, stream);
}

}  // namespace fa
