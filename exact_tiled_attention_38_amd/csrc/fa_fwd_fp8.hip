// Exact tiled attention forward on fp8 (e4m3) Q, K, V with per-tensor
// dequantisation factors; bf16 O and fp32 lse out; gfx950, d = 128.
//
// The method is the forward of fa_fwd_bf16.hip ("Attention and KV
// Compression", "Tiling and online softmax"; "FlashAttention — how 100K-token
// attention fits in memory", "Online softmax intuition") on narrower numbers,
// the refinement named in "What it does and does not change". The attention
// computed is the exact one of the dequantised inputs (code * factor); the
// only rounding beyond fp32 accumulation is that of P to e4m3 before the PV
// product.
//
// Mapping onto CDNA4 (the workgroup, wave and pipeline structure are those of
// the bf16 forward: 8 waves x 32 query rows, direct-to-LDS K/V tile ring,
// lazy reference maximum, upper half of the workgroup shifted by half a
// tile; see there):
//   * Products on v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3 x e4m3, unit
//     scales): K = 64 per instruction, 32 bytes of each operand per lane.
//     The instruction pairs byte j of lane half h of A with byte j of lane
//     half h of B, so the order of the contraction index is ours to choose as
//     long as both operands follow it.
//   * Scores transposed, S^T = K Q^T. Lane m of the A operand loads K row
//     pi(m) = 16 bit2(m) + 4 (m >> 3) + (m & 3) of each 32-key block, so in
//     the result, lane (query n, half h) register i holds key 16h + i: each
//     lane half owns 16 consecutive keys of every 32.
//   * P is rounded to e4m3 two values at a time (v_cvt_pk_fp8_f32) straight
//     into the B operand of O^T += V^T P^T: byte 16kb + i of half h is key
//     32kb + 16h + i. The matching V^T operand (lane = d column, 32 keys in
//     four runs of 8) comes from V's row-major LDS tile by four
//     ds_read_b64_tr_b8 transposed reads.
//   * P headroom: P = 2^(s - m_ref + 4) with the reference moved when a score
//     exceeds it by 2^4, so P <= 2^8 < 448 and values down to 2^-10 of the
//     reference stay normal e4m3 numbers.
//   * Tiles are 64 keys x 128 bytes; 16-byte chunks are XOR-swizzled (K for
//     the permuted 128-bit row reads, V for the transposed reads) so both are
//     free of LDS bank conflicts.
// Scores are kept in log2 units: s2 = s * scale * log2(e) * dq * dk.
#include "fa_device.h"
#include "fa_launch.h"

#ifndef FA_FP8_BN
#define FA_FP8_BN 64
#endif
#ifndef FA_FP8_STAGES
#define FA_FP8_STAGES 8
#endif
#ifndef FA_FP8_PINGPONG
#define FA_FP8_PINGPONG 1
#endif
#ifndef FA_FP8_LA_K
#define FA_FP8_LA_K 2
#endif
// (V operands read ahead of the PV product: 3 of its 4 MFMAs' operands
// before the first, 1.6 % faster than 2 once the tile loads were spread)
#ifndef FA_FP8_LA_V
#define FA_FP8_LA_V 3
#endif

namespace fa {
namespace {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));

#ifndef FA_FP8_SUMCHECK
#define FA_FP8_SUMCHECK 1
#endif
constexpr float kP8Tau = 4.f;    // reference moves when a score exceeds it by 2^4
constexpr float kP8Shift = 4.f;  // P = 2^(s - m_ref + 4) <= 2^8

// Empty asm use of a 32-byte operand, as two 16-byte halves (the host pass
// also checks the constraint, and its 16-byte vector registers fit 128 bits)
__device__ __forceinline__ void pin8(const i32x8_t& x) {
  const u32x4_t lo = {(uint32_t)x[0], (uint32_t)x[1], (uint32_t)x[2], (uint32_t)x[3]};
  const u32x4_t hi = {(uint32_t)x[4], (uint32_t)x[5], (uint32_t)x[6], (uint32_t)x[7]};
  asm volatile("" :: "v"(lo), "v"(hi));
}

__device__ __forceinline__ f32x16_t mfma_f8(i32x8_t a, i32x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// K row loaded by lane m of a 32-key block
__device__ __forceinline__ int krow_of_lane(int m) { return 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3); }
// chunk swizzles of 128-byte rows (two per 256-byte bank line)
__device__ __forceinline__ int fk8(int r) { return ((r >> 1) & 3) | ((r >> 2) & 4); }
__device__ __forceinline__ int fv8(int r) { return ((r >> 1) & 3) << 1; }

template <int NW, int BN, int S>
struct Fp8Cfg {
  static constexpr int D = 128;
  static constexpr int BM = 32 * NW;
  static constexpr int NT = 64 * NW;
  static constexpr int ROWB = D;                  // bytes per K/V row
  static constexpr int TILEB = BN * ROWB;
  static constexpr int CPR = D / 16;              // 16-byte chunks per row
  static constexpr int RPW = 1024 / ROWB;         // rows per wave-wide 1 KB load
  static constexpr int NDMA = TILEB / 1024 / NW;  // wave-wide loads per wave, tile and tensor
  static constexpr int LDS_BYTES = 2 * S * TILEB;
  static constexpr int INFLIGHT = (2 * S - 5) * NDMA;
  static_assert(TILEB % (1024 * NW) == 0, "a tile must split into whole wave-wide loads");
  static_assert(S >= 4 && (S & (S - 1)) == 0 && INFLIGHT <= 63, "stages");
  static_assert(BN % 64 == 0, "a tile is a whole number of 64-key MFMA steps");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS capacity");
};

template <int NW, int BN, int S, bool CAUSAL>
__global__ void __launch_bounds__(64 * NW)
fwd_fp8_kernel(const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K, const uint8_t* __restrict__ V,
               uint16_t* __restrict__ O, float* __restrict__ LSE, int N, int n_qtiles, int group, float c2,
               float o_scale) {
  using C = Fp8Cfg<NW, BN, S>;
  constexpr int D = C::D;
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];
  FA_LDS char* lds = (FA_LDS char*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int n = lane & 31;

  // ---- workgroup -> (head, query block): XCD-aware, longest causal first
  const int G = gridDim.x, b = blockIdx.x;
  const int xcd = b & 7, jx = b >> 3, per = G >> 3, rem = G & 7;
  const int logical = xcd * per + min(xcd, rem) + jx;
  int bh, t;
  // Causal, when each XCD's share is whole groups of 4 heads: a group has its
  // blocks go longest first across its 4 heads, so the blocks that start
  // last on an XCD are short ones and its compute units finish together.
  // Unlike the bf16 forward this kernel is not at the power limit, so the
  // shorter tail pays at every size (1.2 % at B8 H32 N16384), although 4
  // heads in flight per XCD miss its L2 more: DRAM reads rise from 2.1 to
  // 5.4 GB per launch there, about 0.6 TB/s.
  if (CAUSAL && rem == 0 && per % (4 * n_qtiles) == 0) {
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
  const size_t kvhead = (size_t)__builtin_amdgcn_readfirstlane(bh / group) * N * D;
  const uint8_t* Qh = Q + head;
  const uint8_t* Kh = K + kvhead;
  const uint8_t* Vh = V + kvhead;

  const int kv_end = CAUSAL ? min(N, q0 + C::BM) : N;
  const int n_tiles = __builtin_amdgcn_readfirstlane((kv_end + BN - 1) / BN);

  // ---- direct-to-LDS tile loads (as in the bf16 forward)
  uint32_t dk_off[C::NDMA], dv_off[C::NDMA];
#pragma unroll
  for (int i = 0; i < C::NDMA; ++i) {
    const int r = (w * C::NDMA + i) * C::RPW + lane / C::CPR;
    const int phys = lane % C::CPR;
    dk_off[i] = r * C::ROWB + 16 * (phys ^ fk8(r));
    dv_off[i] = r * C::ROWB + 16 * (phys ^ fv8(r));
  }
  auto clamp_row = [&](uint32_t off, int lim) {
    return (uint32_t)min((int)(off / C::ROWB), lim) * C::ROWB + (off % C::ROWB);
  };
  auto load_tile = [&](const uint8_t* src, int tt, int slot0, const uint32_t (&off)[C::NDMA]) {
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
      for (int i = 0; i < C::NDMA; ++i) dma16(base, clamp_row(off[i], lim), dst + i * 1024);
    }
  };
  auto load_k = [&](int tt) { load_tile(Kh, tt, 0, dk_off); };
  auto load_v = [&](int tt) { load_tile(Vh, tt, S, dv_off); };
  // The loads of V tile vt (parts 0 .. NDMA-1) and K tile kt (the rest) one
  // wave-wide DMA at a time, so a step can spread them over its PV product
  // (rows always clamped: a no-op below the tail)
  auto load_part = [&](int j, int vt, int kt) {
    const bool is_v = j < C::NDMA;
    const int i = is_v ? j : j - C::NDMA;
    const int tt = is_v ? vt : kt;
    const int slot = (is_v ? S : 0) + (tt & (S - 1));
    const int k0 = min(tt, n_tiles - 1) * BN;
    const char* base = (const char*)((is_v ? Vh : Kh) + (size_t)k0 * D);
    FA_LDS char* dst = lds + slot * C::TILEB + w * C::NDMA * 1024 + i * 1024;
    dma16(base, clamp_row(is_v ? dv_off[i] : dk_off[i], N - 1 - k0), dst);
  };

  // ---- Q^T operand: for 64-wide step c, lane (n, h) holds Q[qrow][64c + 32h .. +31]
  i32x8_t qf[D / 64];
#pragma unroll
  for (int c = 0; c < D / 64; ++c) {
    u32x4_t x0 = {0u, 0u, 0u, 0u}, x1 = {0u, 0u, 0u, 0u};
    if (qrow < N) {
      const uint8_t* src = Qh + (size_t)qrow * D + 64 * c + 32 * h;
      x0 = *(const u32x4_t*)src;
      x1 = *(const u32x4_t*)(src + 16);
    }
    qf[c] = i32x8_t{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
  }
#pragma unroll
  for (int c = 0; c < D / 64; ++c) pin8(qf[c]);

  // LDS read offsets. K (row reads): row pi(n) (+32 kb), logical chunks
  // 4c + 2h and 4c + 2h + 1 at koff[x] ^ 64c. V (transposed reads): row
  // 16h + (lane & 15) / 2 (+ 8 per read, + 32 per key block), logical chunk
  // 2j + bit 4 of the lane, at voff ^ 32j.
  const int krow = krow_of_lane(n);
  const int koff0 = krow * C::ROWB + 16 * ((2 * h) ^ fk8(krow));
  const int koff1 = krow * C::ROWB + 16 * ((2 * h + 1) ^ fk8(krow));
  const int vrow = 16 * h + ((lane & 15) >> 1);
  const int voff = vrow * C::ROWB + 16 * (((lane >> 4) & 1) ^ fv8(vrow)) + 8 * (lane & 1);

  float m_run = -INFINITY;  // reference maximum of s2 for row qrow
  float l_run = 0.f;        // sum of 2^(s2 - m_run + 4) over this lane's keys
  f32x16_t acc[D / 32];     // O^T block: lane holds O[qrow][32j + 8(i/4) + 4h + i%4]
#pragma unroll
  for (int j = 0; j < D / 32; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[j][i] = 0.f;

  auto k_base = [&](int buf) { return (int)(uintptr_t)(lds + buf * C::TILEB); };
  auto v_base = [&](int buf) { return (int)(uintptr_t)(lds + (S + buf) * C::TILEB); };

  constexpr int KQ = BN / 32 * D / 64;  // score MFMAs per tile
  constexpr int KP = D / 32 * BN / 64;  // PV MFMAs per tile
  constexpr int VPS = (BN / 2) / KQ;    // softmax values per lane per score MFMA
  static_assert(VPS % 2 == 0, "slicing");
  constexpr int LA_K = FA_FP8_LA_K < KQ ? FA_FP8_LA_K : KQ;
  constexpr int LA_V = FA_FP8_LA_V < KP ? FA_FP8_LA_V : KP;

  // score MFMA i: 64-wide d step c = i / (BN/32), key block kb = i % (BN/32)
  auto kread = [&](int kb0, int i) {
    const int c = i / (BN / 32), kb = i % (BN / 32);
    const FA_LDS char* p0 = (FA_LDS char*)(uintptr_t)((kb0 + koff0) ^ (64 * c)) + kb * 32 * C::ROWB;
    const FA_LDS char* p1 = (FA_LDS char*)(uintptr_t)((kb0 + koff1) ^ (64 * c)) + kb * 32 * C::ROWB;
    const u32x4_t a = *(const FA_LDS u32x4_t*)p0;
    const u32x4_t bb = *(const FA_LDS u32x4_t*)p1;
    return i32x8_t{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)bb[0], (int)bb[1], (int)bb[2], (int)bb[3]};
  };
  // PV MFMA k: d block j = k / (BN/64), 64-key step kc = k % (BN/64); four
  // transposed reads of 8 keys: key runs 16h + {0, 8} and 32 + 16h + {0, 8}
  auto vread = [&](int vb0, int k) {
    const int j = k / (BN / 64), kc = k % (BN / 64);
    const int base = (vb0 + voff + 64 * kc * C::ROWB) ^ (32 * j);
    i32x2_t r[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const int rows = 32 * (tt >> 1) + 8 * (tt & 1);
      r[tt] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((FA_LDS i32x2_t*)(uintptr_t)(base + rows * C::ROWB));
    }
    return i32x8_t{r[0][0], r[0][1], r[1][0], r[1][1], r[2][0], r[2][1], r[3][0], r[3][1]};
  };

  // causal / tail mask of the tile starting at key k0: register i of key
  // block kb holds key k0 + 32kb + 16h + i
  auto mask = [&](int k0, f32x16_t (&s)[BN / 32]) {
    const int lim = (CAUSAL ? min(qrow, N - 1) : N - 1) - k0 - 16 * h;
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (32 * kb + i > lim) s[kb][i] = -INFINITY;
  };
  auto row_max = [&](const f32x16_t (&s)[BN / 32]) {
    float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
    for (int f = 2; f < BN / 2; f += 2) mx = max3(mx, s[f >> 4][f & 15], s[f >> 4][(f + 1) & 15]);
    return halves_max(mx);
  };
  auto qk = [&](int kb0, f32x16_t (&s)[BN / 32]) {
#pragma unroll
    for (int i = 0; i < KQ; ++i) {
      const int c = i / (BN / 32), kb = i % (BN / 32);
      const f32x16_t z = {};
      s[kb] = mfma_f8(kread(kb0, i), qf[c], c == 0 ? z : s[kb]);
    }
  };

  // scores of the next tile interleaved with the softmax of the current one;
  // P goes to e4m3, value f (= 16 kb + i) of the lane to byte f % 32 of
  // 64-key step f / 32
  auto qk_softmax = [&](int kb0, float m_use, const f32x16_t (&s_cur)[BN / 32], f32x16_t (&s_nxt)[BN / 32],
                        i32x8_t (&p)[BN / 64]) {
    i32x8_t kr[KQ];
#pragma unroll
    for (int i = 0; i < LA_K; ++i) kr[i] = kread(kb0, i);
    float lsum = 0.f;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < KQ; ++i) {
      if (i + LA_K < KQ) kr[i + LA_K] = kread(kb0, i + LA_K);
      const int c = i / (BN / 32), kb = i % (BN / 32);
      const f32x16_t z = {};
      s_nxt[kb] = mfma_f8(kr[i], qf[c], c == 0 ? z : s_nxt[kb]);
#pragma unroll
      for (int e = 0; e < VPS; e += 2) {
        const int f = i * VPS + e;
        const float p0 = exp2_fast(fmaf(s_cur[f >> 4][f & 15], c2, -m_use));
        const float p1 = exp2_fast(fmaf(s_cur[f >> 4][(f + 1) & 15], c2, -m_use));
        lsum += p0 + p1;
        const int kc = f >> 5, byte = f & 31;
        if (byte & 2) p[kc][byte >> 2] = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, p[kc][byte >> 2], true);
        else p[kc][byte >> 2] = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, p[kc][byte >> 2], false);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 0; i < BN / 64; ++i) pin8(p[i]);
    asm volatile("" :: "v"(lsum));
    return lsum;
  };
  auto rescale = [&](float alpha) {
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
      for (int j = 0; j < D / 32; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[j][e] *= alpha;
    }
  };
  // acc += P V, with the step's tile loads (V tile vt, K tile kt; none if
  // vt < 0) issued one every KP / (2 NDMA) matrix instructions: issued at
  // the step's start, every wave's loads would queue in the address unit
  // at once while the SIMDs idle (9.49 -> 9.02 ms at the causal N = 16384
  // fp8 workload, bitwise unchanged)
  constexpr int LD_EVERY = KP / (2 * C::NDMA);
  static_assert(LD_EVERY >= 1 && KP % (2 * C::NDMA) == 0, "load spread");
  auto pv = [&](int vb0, const i32x8_t (&p)[BN / 64], int vt, int kt) {
    i32x8_t vr[KP];
#pragma unroll
    for (int k = 0; k < LA_V; ++k) vr[k] = vread(vb0, k);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < KP; ++k) {
      if (k + LA_V < KP) vr[k + LA_V] = vread(vb0, k + LA_V);
      if (k % LD_EVERY == LD_EVERY / 2 && vt >= 0) load_part(k / LD_EVERY, vt, kt);
      const int j = k / (BN / 64), kc = k % (BN / 64);
      acc[j] = mfma_f8(vr[k], p[kc], acc[j]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- pipeline: the same ring, waits and step order as the bf16 forward
#pragma unroll
  for (int tt = 0; tt + 2 < S; ++tt) {
    load_k(tt);
    load_v(tt);
  }
  load_k(S - 2);
  load_k(S - 1);
  wait_loads_and_barrier<C::INFLIGHT>();

  f32x16_t sA[BN / 32], sB[BN / 32];
  i32x8_t pA[BN / 64], pB[BN / 64];
#pragma unroll
  for (int i = 0; i < BN / 64; ++i) pA[i] = pB[i] = i32x8_t{0, 0, 0, 0, 0, 0, 0, 0};
  qk(k_base(0), sA);
  // step 0 loads K(S) into slot 0, which every wave has just read: wait
  // until they all have
  lds_barrier();
  if constexpr (FA_FP8_SUMCHECK) {
    // key 0 is visible to every row: the first tile's masked maximum is a
    // finite initial reference (step_head(0) applies the same mask again)
    if ((CAUSAL && BN - 1 > row0) || BN > N) mask(0, sA);
    m_run = row_max(sA) * c2;
  }

  // (the step's loads, V(u+S-2) and K(u+S), go out during its PV product)
  auto step_head = [&](int u, f32x16_t (&s_cur)[BN / 32], int& kb0, int& vb0, int v_tile, float& m_use,
                       float& alpha) {
    const int k0 = u * BN;
    if ((CAUSAL && k0 + BN - 1 > row0) || k0 + BN > N) mask(k0, s_cur);
    kb0 = k_base((u + 1) & (S - 1));
    vb0 = v_base(v_tile & (S - 1));
    asm volatile("" : "+v"(kb0), "+v"(vb0));
    if constexpr (FA_FP8_SUMCHECK) {
      // the reference only moves in check() below
      m_use = m_run - kP8Shift;
      alpha = 1.f;
      return;
    }
    const float mx = row_max(s_cur);
    const bool move = __builtin_amdgcn_ballot_w64(mx * c2 > m_run + kP8Tau) != 0;
    const float m_new = move ? fmaxf(m_run, mx * c2) : m_run;
    m_use = (m_new == -INFINITY) ? 0.f : m_new - kP8Shift;
    alpha = exp2_fast((m_run - kP8Shift) - m_use);
    m_run = m_new;
  };
  // Row-sum check: P of a tile is formed with the row's current reference;
  // a lane's share of the tile's row sum of at most 2^8 bounds every P by
  // 2^8 (as the lazy rule does; e4m3 holds up to 448). Otherwise (rare: a
  // score well above the reference) the wave takes the tile's row maxima,
  // moves each row's reference to its maximum, rescales l and acc, and forms
  // the tile's P again. The reference is always a score the row has seen,
  // so the largest P of a row is at least 2^4, as with the lazy rule.
  auto check = [&](const f32x16_t (&s_cur)[BN / 32], i32x8_t (&p)[BN / 64], float& lsum) {
    if constexpr (FA_FP8_SUMCHECK) {
      // (on the bit pattern: the sum is never negative, so every value
      // above 2^8 (0x43800000), +inf and every NaN compare above it as
      // unsigned integers; this file is built without NaN semantics, and
      // the empty asm makes the pattern an opaque integer, so the compiler
      // cannot turn the test back into a float compare)
      uint32_t lbits = __float_as_uint(lsum);
      asm volatile("" : "+v"(lbits));
      if (__builtin_amdgcn_ballot_w64(lbits > 0x43800000u)) {
        const float mx = row_max(s_cur);
        const float m_new = fmaxf(m_run, mx * c2);
        const float a = exp2_fast(m_run - m_new);
        m_run = m_new;
        l_run *= a;
#pragma unroll
        for (int j = 0; j < D / 32; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[j][e] *= a;
        const float m_use = m_new - kP8Shift;
        lsum = 0.f;
#pragma unroll
        for (int f = 0; f < BN / 2; f += 2) {
          const float p0 = exp2_fast(fmaf(s_cur[f >> 4][f & 15], c2, -m_use));
          const float p1 = exp2_fast(fmaf(s_cur[f >> 4][(f + 1) & 15], c2, -m_use));
          lsum += p0 + p1;
          const int kc = f >> 5, byte = f & 31;
          if (byte & 2) p[kc][byte >> 2] = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, p[kc][byte >> 2], true);
          else p[kc][byte >> 2] = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, p[kc][byte >> 2], false);
        }
      }
    }
  };
  auto step_lo = [&](int u, f32x16_t (&s_cur)[BN / 32], f32x16_t (&s_nxt)[BN / 32], i32x8_t (&p)[BN / 64]) {
    int kb0, vb0;
    float m_use, alpha;
    step_head(u, s_cur, kb0, vb0, u, m_use, alpha);
    float lsum = qk_softmax(kb0, m_use, s_cur, s_nxt, p);
    check(s_cur, p, lsum);
    l_run = l_run * alpha + lsum;
    rescale(alpha);
    pv(vb0, p, u + S - 2, u + S);
    wait_loads_and_barrier<C::INFLIGHT>();
  };
  auto step_hi = [&](int u, f32x16_t (&s_cur)[BN / 32], f32x16_t (&s_nxt)[BN / 32], i32x8_t (&p_cur)[BN / 64],
                     const i32x8_t (&p_prev)[BN / 64], bool first) {
    int kb0, vb0;
    float m_use, alpha;
    step_head(u, s_cur, kb0, vb0, u - 1, m_use, alpha);
    if (!first) {
      pv(vb0, p_prev, u + S - 2, u + S);
    } else {
#pragma unroll
      for (int j = 0; j < 2 * C::NDMA; ++j) load_part(j, u + S - 2, u + S);
    }
    float lsum = qk_softmax(kb0, m_use, s_cur, s_nxt, p_cur);
    check(s_cur, p_cur, lsum);
    l_run = l_run * alpha + lsum;
    rescale(alpha);
    wait_loads_and_barrier<C::INFLIGHT>();
  };

  const int n_steps = (n_tiles + 1) & ~1;
  if (!FA_FP8_PINGPONG || w < NW / 2) {
    for (int u = 0; u < n_steps; u += 2) {
      step_lo(u, sA, sB, pA);
      step_lo(u + 1, sB, sA, pB);
    }
  } else {
    step_hi(0, sA, sB, pA, pB, true);
    for (int u = 1; u + 1 < n_steps; u += 2) {
      step_hi(u, sB, sA, pB, pA, false);
      step_hi(u + 1, sA, sB, pA, pB, false);
    }
    step_hi(n_steps - 1, sB, sA, pB, pA, false);
    pv(v_base((n_steps - 1) & (S - 1)), pB, -1, 0);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- epilogue: O = v_descale * acc / l, lse = ln(2) * (m_ref - 4 + log2 l)
  if (qrow < N) {
    const float l_tot = halves_sum(l_run);
    const float inv = o_scale / l_tot;
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
    if (h == 0) LSE[(size_t)bh * N + qrow] = (m_run - kP8Shift + log2_fast(l_tot)) * kLn2;
  }
}

template <int NW, int BN, int S, bool CAUSAL>
hipError_t launch(const void* q, const void* k, const void* v, void* o, float* lse, const Problem& p,
                  const Fp8Scales& sc, hipStream_t stream) {
  using C = Fp8Cfg<NW, BN, S>;
  const int n_qtiles = (p.N + C::BM - 1) / C::BM;
  const long long grid = (long long)p.B * p.H * n_qtiles;
  const float c2 = p.scale * kLog2e * sc.q * sc.k;
  hipLaunchKernelGGL((fwd_fp8_kernel<NW, BN, S, CAUSAL>), dim3((unsigned)grid), dim3(C::NT), 0, stream,
                     (const uint8_t*)q, (const uint8_t*)k, (const uint8_t*)v, (uint16_t*)o, lse, p.N, n_qtiles,
                     p.group(), c2, sc.v);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, const Problem& p,
                          const Fp8Scales& sc, hipStream_t stream) {
  static_assert(Fp8Cfg<8, FA_FP8_BN, FA_FP8_STAGES>::BM == kFwdRowsPerBlock, "grid-size limit assumes 256-row blocks");
  return p.causal ? launch<8, FA_FP8_BN, FA_FP8_STAGES, true>(q, k, v, o, lse, p, sc, stream)
                  : launch<8, FA_FP8_BN, FA_FP8_STAGES, false>(q, k, v, o, lse, p, sc, stream);
}

}  // namespace fa
