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
//     operand is read from V's row-major LDS tile with ds_read_b64_tr_b16.
//     The contraction index order inside each 16-key MFMA step follows the
//     score registers' key order, which the two transposed reads reproduce
//     (rows 4h..4h+3 and 8+4h..8+4h+3 of each 16-key group).
//   * K and V tiles (BN keys) move from HBM to LDS with direct-to-LDS 16-byte
//     loads (global_load_lds_dwordx4; each wave-wide load fills 1 KB of
//     consecutive LDS), so no registers or LDS-store instructions stage them.
//     Rows are unpadded; the 16-byte chunks of a row are XOR-swizzled by a
//     function of the row so that both the 128-bit K reads (16 rows, one
//     chunk column) and the transposed V reads (4 rows x 64 bytes) hit 64
//     distinct banks. A lane of the wave-wide load fetches the global chunk
//     that belongs at its LDS slot.
//   * Ring of S K tiles and S V tiles in LDS, one barrier per tile. Every
//     step issues the loads of tiles several steps ahead and waits (vmcnt)
//     only for the ones the next step reads. The loads are inline assembly,
//     so the compiler neither orders nor counts them; the waits are explicit.
//   * A step is straight-line code with an explicit instruction schedule
//     (sched_barrier slices): the scores of tile u+1 run on the matrix cores
//     while the vector unit runs the softmax update of tile u (exponentials,
//     row sum, bf16 rounding of P) and the accumulator rescale by alpha, one
//     slice per matrix instruction; then P(u) V(u) accumulates. LDS reads
//     are issued a few matrix instructions ahead.
//   * Waves w and w + 4 share a SIMD. The upper half of the workgroup runs
//     the same steps shifted by half a tile (PV of the previous tile first),
//     so one wave of a SIMD feeds the matrix core while the other runs its
//     exponentials.
//   * Exactness needs one reference per row used for P, l, acc and lse
//     alike, not the true running maximum. A block first runs a pass in
//     which each row's reference is the maximum of its scores in the first
//     tile and never moves: no per-tile row maximum at all. The row sums the
//     softmax forms anyway bound P: if a lane's share of a tile's row sum
//     exceeds 2^40 (or is not finite), or an accumulator value is not finite
//     at the end, the wave flags it, and the workgroup reruns the block in
//     the checked pass. Checked pass: the reference is lazy,
//     it moves (and the accumulator is rescaled, in a branch taken by the
//     whole wave) only when a score of the wave's rows exceeds its row's
//     reference by more than 2^8, so P <= 2^8 and the per-tile rescale of
//     the accumulator disappears from almost every step.
//   * Every wave runs every tile of the workgroup's key range: a tile wholly
//     after a wave's rows is masked entirely (alpha = 1, P = 0, acc and l
//     unchanged), which keeps the loop free of branches around the work.
//   * Causal: the key range of a query block ends at its last row; only tiles
//     touching the diagonal or the ragged tail (keys >= N) are masked. The
//     loads go through a buffer resource whose range ends at key N, so
//     tail rows arrive as zeros (no per-lane clamp) and are masked.
//   * Grid order: workgroups are dispatched round-robin over the 8 XCDs; the
//     block index is remapped so each XCD works through whole heads (K/V of a
//     head stay in that XCD's L2), longest causal query blocks first.
// Scores are kept in log2 units: s2 = s * scale * log2(e), so exp is v_exp_f32.
#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"

#ifndef FA_FWD_BN
#define FA_FWD_BN 64
#endif
#ifndef FA_FWD_STAGES
#define FA_FWD_STAGES 4
#endif
// Tuning switches (all settings compute the same result up to rounding):
// 1: the accumulator rescale is spread over the score/softmax slices (always
// done); 0: it is a separate block skipped when no row's reference moved
#ifndef FA_FWD_RESCALE_IN_SLICES
#define FA_FWD_RESCALE_IN_SLICES 0
#endif
// 1: the upper half of the workgroup runs its steps half a tile shifted
#ifndef FA_FWD_PINGPONG
#define FA_FWD_PINGPONG 1
#endif
// > 0: the reference maximum of a row only moves when some row of the wave
// sees a score above its reference by more than this (log2 units)
#ifndef FA_FWD_LAZY_TAU
#define FA_FWD_LAZY_TAU 8
#endif
// > 0: issue priority of a wave while it runs its scores + softmax slices
// (back to 0 after them, so its PV products and the other wave's run at 0)
#ifndef FA_FWD_PRIO_QK
#define FA_FWD_PRIO_QK 1
#endif
// 1: every block first runs a pass with a fixed per-row reference and a
// row-sum bound check, and falls back to the checked lazy reference only
// where the bound fails
#ifndef FA_FWD_FAST_PASS
#define FA_FWD_FAST_PASS 1
#endif

// Race check (built as a separate library, never the product): 1 waits for
// every outstanding tile load at each step's end instead of only the ones the
// next step reads, and adds a workgroup barrier after each LDS read phase
// (scores and PV). The arithmetic is the same, so its results must equal the
// pipelined kernel's bit for bit; a tile read before its load landed, or
// overwritten while another wave still read it, would show as a difference.
#ifndef FA_SAFE_SYNC
#define FA_SAFE_SYNC 0
#endif

namespace fa {
namespace {

// end of a step: this wave's loads of the tiles the next step reads are in
// LDS (all of them, in the race-check build), then the workgroup barrier
template <int INFLIGHT>
__device__ __forceinline__ void step_sync() {
  if constexpr (FA_SAFE_SYNC) wait_loads_and_barrier<0>();
  else wait_loads_and_barrier<INFLIGHT>();
}
// end of an LDS read phase: nothing, or (race-check build) a barrier after
// this wave's LDS reads completed
__device__ __forceinline__ void phase_sync() {
  if constexpr (FA_SAFE_SYNC) lds_barrier();
}

template <int D, int NW, int BN, int S>
struct FwdCfg {
  static constexpr int BM = 32 * NW;              // query rows per workgroup
  static constexpr int NT = 64 * NW;              // threads
  static constexpr int ROWB = 2 * D;              // bytes per K/V row in LDS (unpadded)
  static constexpr int TILEB = BN * ROWB;         // bytes per K (or V) tile
  static constexpr int CPR = D / 8;               // 16-byte chunks per row
  static constexpr int RPW = 1024 / ROWB;         // rows filled by one wave-wide 1 KB load
  static constexpr int NDMA = TILEB / 1024 / NW;  // wave-wide loads per wave, per tile and tensor
  static constexpr int STAGES = S;                // K and V tiles resident in LDS (ring)
  static constexpr int LDS_BYTES = 2 * S * TILEB; // K slots 0..S-1, then V slots 0..S-1
  // DMAs a wave may leave in flight at the end of a step: the tiles issued
  // after the ones the next step reads (see the pipeline below)
  static constexpr int INFLIGHT = (2 * S - 5) * NDMA;
  static_assert(TILEB % (1024 * NW) == 0, "a tile must split into whole wave-wide loads");
  static_assert(S >= 4 && (S & (S - 1)) == 0 && INFLIGHT <= 63, "stages: power of two >= 4, vmcnt range");
  static_assert(NW % 2 == 0, "two halves of the workgroup share the SIMDs");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS capacity");
  static_assert(BN % 32 == 0 && (D == 64 || D == 128), "tile shape");
};

// Key-block selection of the block-sparse forward, in compressed-row form:
// the key blocks (of BN keys) of query block r (of BM rows; r counts over
// (b, h, block)) are cols[row_ptr[r] .. row_ptr[r + 1]). Offsets and block
// indices are clamped into range, so no list content can send a load out of
// bounds.
struct BlockList {
  const int* row_ptr;
  const int* cols;
  int nnz;
};

// (8 waves per compute unit: one 8-wave workgroup, or two of 4 waves)
template <int D, int NW, int BN, int S, bool CAUSAL, bool SPARSE>
__global__ void __launch_bounds__(64 * NW, 8 / NW)
fwd_bf16_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                float* __restrict__ LSE, int N, int n_qtiles, int group, float c2,
                const int* __restrict__ sel_row_ptr, const int* __restrict__ sel_cols, int sel_nnz) {
  using C = FwdCfg<D, NW, BN, S>;
  constexpr bool FAST = FA_FWD_FAST_PASS;
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];
  __shared__ int redo_flag;
  FA_LDS char* lds = (FA_LDS char*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // (ordered before any wave's report by the barriers of the first pass)
  if (FAST && tid == 0) redo_flag = 0;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, held in a scalar register
  const int h = lane >> 5;  // which 16 of each 32 keys this lane holds
  const int n = lane & 31;  // this lane's query row within the wave

  // ---- workgroup -> (head, query block): XCD-aware, longest causal first
  const int G = gridDim.x, b = blockIdx.x;
  const int xcd = b & 7, jx = b >> 3, per = G >> 3, rem = G & 7;
  const int logical = xcd * per + min(xcd, rem) + jx;
  // (integer division runs on the vector unit; the results are uniform, so
  // move them back to scalar registers and keep all tile bookkeeping scalar)
  int bh, t;
  // Causal dense, when each XCD's share is 4 or 8 whole heads: a group of 4
  // heads has its blocks go longest first across the 4 rather than head by
  // head, so the blocks that start last on an XCD are short ones and its
  // compute units finish together. (With more heads per XCD the idle tail is
  // a small part of the time, and keeping one head's keys and values in
  // flight per XCD lets its L2 hold them: with 4 heads interleaved the
  // forward's DRAM reads double.)
  if (CAUSAL && !SPARSE && rem == 0 && per % (4 * n_qtiles) == 0 && per <= 8 * n_qtiles) {
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
  const uint16_t* Qh = Q + head;
  const uint16_t* Kh = K + kvhead;
  const uint16_t* Vh = V + kvhead;

  // Key tiles: dense, tiles 0 .. n_tiles-1 (causal: up to the block's last
  // row); block-sparse, the listed key blocks in list order (the online
  // softmax does not depend on the order).
  int n_tiles, sel_base = 0;
  if constexpr (SPARSE) {
    const int r = bh * n_qtiles + t;
    // (read-only, uniform: scalar loads, which do not wait on the tile loads)
    const int beg = min(max(sel_row_ptr[r], 0), sel_nnz);
    const int end = min(max(sel_row_ptr[r + 1], beg), sel_nnz);
    sel_base = __builtin_amdgcn_readfirstlane(beg);
    n_tiles = __builtin_amdgcn_readfirstlane(end - beg);
  } else {
    const int kv_end = CAUSAL ? min(N, q0 + C::BM) : N;
    n_tiles = __builtin_amdgcn_readfirstlane((kv_end + BN - 1) / BN);
  }
  // first key of tile t (tiles past the last repeat the last one); for the
  // block-sparse list in two parts, the read (list_entry) and the clamp
  // into range (entry_key), so a read can be issued well before its use
  auto list_entry = [&](int t) { return sel_cols[sel_base + min(t, n_tiles - 1)]; };
  auto entry_key = [&](int e) { return min(max(e, 0), (N - 1) / BN) * BN; };
  auto tile_key = [&](int t) {
    if constexpr (SPARSE) return entry_key(list_entry(t));
    else return min(t, n_tiles - 1) * BN;
  };
  if constexpr (SPARSE) {
    if (n_tiles == 0) {  // nothing selected: no key is visible to these rows
      if (qrow < N) {
        uint16_t* Orow = O + head + (size_t)qrow * D;
#pragma unroll
        for (int c = 0; c < D / 8; ++c) *(u32x2_t*)(Orow + 8 * c + 4 * h) = u32x2_t{0u, 0u};
        if (h == 0) LSE[(size_t)bh * N + qrow] = -INFINITY;
      }
      return;
    }
  }

  // ---- direct-to-LDS tile loads. Lane `lane` of wave-wide load i fills the
  // 16-byte LDS slot `lane` of 1 KB block w * NDMA + i of the tile buffer:
  // row r of the tile, physical chunk lane % CPR, so it fetches the global
  // chunk whose swizzled position that is. Byte offsets within a tile
  // (row r * ROWB + chunk * 16) are kept per lane; the tile base is scalar.
  uint32_t dk_off[C::NDMA], dv_off[C::NDMA];
#pragma unroll
  for (int i = 0; i < C::NDMA; ++i) {
    const int r = (w * C::NDMA + i) * C::RPW + lane / C::CPR;
    const int phys = lane % C::CPR;
    dk_off[i] = r * C::ROWB + 16 * (phys ^ kswz<D>(r));
    dv_off[i] = r * C::ROWB + 16 * (phys ^ vswz<D>(r));
  }
  // rows past the last key (tail tile) read as zeros through the buffer
  // resource's range; the mask excludes them
  // Tile t goes to ring slot t % S. Past the last tile the loads repeat the
  // last tile into the (unused) slot, so every step issues the same number
  // of loads and the wait count below is a constant.
  auto load_tile = [&](const uint16_t* src, int t, int slot0, const uint32_t (&off)[C::NDMA], int k0) __attribute__((always_inline)) {
    const int slot = slot0 + (t & (S - 1));
    const i32x4_t rsrc = buffer_rsrc(src + (size_t)k0 * D, (uint32_t)min(N - k0, BN) * C::ROWB);
    FA_LDS char* dst = lds + slot * C::TILEB + w * C::NDMA * 1024;
#pragma unroll
    for (int i = 0; i < C::NDMA; ++i) dma16_buf(rsrc, off[i], dst + i * 1024);
  };
  auto load_k = [&](int t, int k0) { load_tile(Kh, t, 0, dk_off, k0); };
  auto load_v = [&](int t, int k0) { load_tile(Vh, t, S, dv_off, k0); };
  // The same loads one wave-wide DMA at a time, so a step can spread them
  // over its matrix instructions: part j < NDMA is V tile vt's load j, the
  // rest K tile kt's.
  auto load_part = [&](int j, int vt, int vk0, int kt, int kk0) __attribute__((always_inline)) {
    const bool is_v = j < C::NDMA;
    const int i = is_v ? j : j - C::NDMA;
    const int k0 = is_v ? vk0 : kk0;
    const int slot = (is_v ? S : 0) + ((is_v ? vt : kt) & (S - 1));
    const i32x4_t rsrc = buffer_rsrc((is_v ? Vh : Kh) + (size_t)k0 * D, (uint32_t)min(N - k0, BN) * C::ROWB);
    FA_LDS char* dst = lds + slot * C::TILEB + w * C::NDMA * 1024 + i * 1024;
    dma16_buf(rsrc, is_v ? dv_off[i] : dk_off[i], dst);
  };

  // ---- Q^T operand: lane holds Q[qrow][16c + 8h .. +7]
  bf16x8_t qf[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    u32x4_t x = {0u, 0u, 0u, 0u};
    if (qrow < N) x = *(const u32x4_t*)(Qh + (size_t)qrow * D + 16 * c + 8 * h);
    qf[c] = __builtin_bit_cast(bf16x8_t, x);
  }
  // take delivery of Q before the tile loads start, so the wait for Q does
  // not also wait for the tiles queued behind it
#pragma unroll
  for (int c = 0; c < D / 16; ++c) asm volatile("" :: "v"(qf[c]));

  // LDS read offsets (bytes, within a tile buffer).
  // K: row kb*32 + n, logical chunk 2c + h, at koff0 ^ (32 c): the swizzle
  // only permutes the chunk index bits above the lowest one, so the offset
  // for d-chunk c is one XOR away from that of chunk 0.
  const int koff0 = n * C::ROWB + 16 * (h ^ kswz<D>(n));
  // V (transposed reads): row 4h + q, q = (lane >> 2) & 3 (plus a multiple
  // of 16, and 8 more for the upper half); columns 32j + 16x + 4(lane & 3),
  // x = (lane >> 4) & 1, at voff0 ^ (64 j).
  const int tr_row = 4 * h + ((lane >> 2) & 3);
  const int tr_chunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int voff0 = tr_row * C::ROWB + 16 * (tr_chunk ^ vswz<D>(tr_row)) + 8 * (lane & 1);

  float m_run = -INFINITY;  // reference maximum of s2 for row qrow (see step_head, run)
  float l_run = 0.f;        // running sum of 2^(s2 - m_run) over this lane's keys
  f32x16_t acc[D / 32];     // O^T block: lane holds O[qrow][32j + 8(i/4) + 4h + i%4]
#pragma unroll
  for (int j = 0; j < D / 32; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[j][i] = 0.f;

  // LDS byte addresses of this lane's K row (chunk 0) and V row (d-block 0)
  // in ring slot `buf`: a slot base is a multiple of 1 KB, so the XOR on bits
  // 5..7 that selects a chunk commutes with adding it.
  auto k_addr = [&](int buf) { return (int)(uintptr_t)(lds + buf * C::TILEB) + koff0; };
  auto v_addr = [&](int buf) { return (int)(uintptr_t)(lds + (S + buf) * C::TILEB) + voff0; };

  // S^T = K Q^T for the BN keys of the K tile at LDS address kb0
  auto qk = [&](int kb0, f32x16_t (&s)[BN / 32]) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const FA_LDS char* kp = (FA_LDS char*)(uintptr_t)(kb0 ^ (32 * c));
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb) {
        const bf16x8_t a = *(const FA_LDS bf16x8_t*)(kp + kb * 32 * C::ROWB);
        s[kb] = mfma_32x32x16(a, qf[c], s[kb]);
      }
    }
  };

  // causal / tail mask of the tile starting at key k0: key j is kept iff
  // j <= qrow (causal) and j < N, i.e. (j - k0 - 4h) <= lim below
  auto mask = [&](int k0, f32x16_t (&s)[BN / 32]) __attribute__((always_inline)) {
    const int lim = (CAUSAL ? min(qrow, N - 1) : N - 1) - k0 - 4 * h;
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (kb * 32 + 8 * (i >> 2) + (i & 3) > lim) s[kb][i] = -INFINITY;
  };

  // online softmax update of one tile: new max, P (bf16), l, acc rescale.
  // Split in two so the row max can be issued ahead of the matrix work.
  // (a chain of three-input maxima: one instruction per two scores)
  auto row_max = [&](const f32x16_t (&s)[BN / 32]) __attribute__((always_inline)) {
    float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
    for (int f = 2; f < BN / 2; f += 2) mx = max3(mx, s[f >> 4][f & 15], s[f >> 4][(f + 1) & 15]);
    return halves_max(mx);
  };

  // ---- the step's pieces, each an explicit instruction schedule: LDS reads
  // run a few matrix instructions ahead, and every slice ends in a
  // scheduling barrier so the compiler keeps the order (it schedules freely
  // within a slice).
  constexpr int KQ = BN / 32 * D / 16;   // score MFMAs per tile
  constexpr int KP = BN / 16 * D / 32;   // PV MFMAs per tile
  constexpr int VPS = (BN / 2) / KQ;     // softmax values per lane per score MFMA
#ifndef FA_FWD_LA_K
#define FA_FWD_LA_K 3
#endif
#ifndef FA_FWD_LA_V
#define FA_FWD_LA_V 2
#endif
  constexpr int LA_K = FA_FWD_LA_K, LA_V = FA_FWD_LA_V;  // read lookahead (MFMAs)
  static_assert(VPS % 2 == 0, "slicing");
  // score MFMA i: d-chunk c = i / (BN/32), key block kb = i % (BN/32)
  auto kread = [&](int kb0, int i) {
    const int c = i / (BN / 32), kb = i % (BN / 32);
    return *(const FA_LDS bf16x8_t*)((FA_LDS char*)(uintptr_t)(kb0 ^ (32 * c)) + kb * 32 * C::ROWB);
  };
  // PV MFMA k: d-block j = k / (BN/16), 16-key group kc = k % (BN/16)
  auto vread = [&](int vb0, int k) {
    const int j = k / (BN / 16), kc = k % (BN / 16);
    const FA_LDS char* vp = (FA_LDS char*)(uintptr_t)(vb0 ^ (64 * j)) +
                            ((kc >> 1) * 32 + 16 * (kc & 1)) * C::ROWB;
    const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((FA_LDS bf16x4_t*)vp);
    const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((FA_LDS bf16x4_t*)(vp + 8 * C::ROWB));
    return concat8(lo, hi);
  };

  // Scores of the next tile (K at kb0) on the matrix cores, interleaved
  // slice by slice with the softmax of the current tile on the vector unit
  // (exponentials, row sum, bf16 rounding of P). Returns the row sum.
  // kpre: the first LA_K K operands, already read (or null: read here).
  // vout: if not null, the last slices also read the first LA_V V operands
  // of the PV product at vb_next that follows, so it need not wait for LDS.
  auto qk_softmax = [&](int kb0, float m_use, float alpha, const f32x16_t (&s_cur)[BN / 32],
                        f32x16_t (&s_nxt)[BN / 32], bf16x8_t (&p)[BN / 16], const bf16x8_t* kpre,
                        int vb_next, bf16x8_t* vout) __attribute__((always_inline)) {
    bf16x8_t kr[KQ];
#pragma unroll
    for (int i = 0; i < LA_K; ++i) kr[i] = kpre ? kpre[i] : kread(kb0, i);
    float lsum = 0.f;
    // The two waves of a SIMD contend for its issue port and matrix core, and
    // a wave issues in order: while this one interleaves score MFMAs with
    // softmax work, the other is usually in its PV run of back-to-back
    // MFMAs. Winning that arbitration lets this wave's MFMA go as soon as
    // the matrix core is free, so the vector work behind it is not held up
    // (2-3 % on the causal N = 16384 forward; results unchanged).
    if constexpr (FA_FWD_PRIO_QK > 0) __builtin_amdgcn_s_setprio(FA_FWD_PRIO_QK);
    __builtin_amdgcn_sched_barrier(0);
    // softmax values of slice i (exponentials, row sum, bf16 rounding)
    auto softmax_slice = [&](int i) __attribute__((always_inline)) {
#pragma unroll
      for (int e = 0; e < VPS; e += 2) {
        const int f = i * VPS + e;  // flat index of the value within the lane's BN/2
        const float p0 = exp2_fast(fmaf(s_cur[f >> 4][f & 15], c2, -m_use));
        const float p1 = exp2_fast(fmaf(s_cur[f >> 4][(f + 1) & 15], c2, -m_use));
        lsum += p0 + p1;
        const bf16x2_t pb = to_bf16x2(p0, p1);
        p[f >> 3][f & 7] = pb[0];
        p[f >> 3][(f + 1) & 7] = pb[1];
      }
    };
#pragma unroll
    for (int i = 0; i < KQ; ++i) {
      if (i + LA_K < KQ) kr[i + LA_K] = kread(kb0, i + LA_K);
      if (vout && i >= KQ - LA_V) vout[i - (KQ - LA_V)] = vread(vb_next, i - (KQ - LA_V));
      const int c = i / (BN / 32), kb = i % (BN / 32);
      if (c == 0) {
        const f32x16_t z = {};
        s_nxt[kb] = mfma_32x32x16(kr[i], qf[c], z);
      } else {
        s_nxt[kb] = mfma_32x32x16(kr[i], qf[c], s_nxt[kb]);
      }
      softmax_slice(i);
      if constexpr (FA_FWD_RESCALE_IN_SLICES) {
        constexpr int per = D / 2 / KQ;  // accumulator values rescaled per slice
#pragma unroll
        for (int e = 0; e < per; ++e) {
          const int g = i * per + e;
          acc[g >> 4][g & 15] *= alpha;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // P and the row sum are complete here: keep the compiler from sinking
    // their computation past the branches that follow
#pragma unroll
    for (int i = 0; i < BN / 16; ++i) asm volatile("" :: "v"(p[i]));
    asm volatile("" :: "v"(lsum));
    if constexpr (FA_FWD_PRIO_QK > 0) __builtin_amdgcn_s_setprio(0);
    return lsum;
  };

  // acc *= alpha, skipped when no row of the wave raised its maximum
  // (alpha = 1 on every lane: multiplying would change nothing)
  auto rescale = [&](float alpha) __attribute__((always_inline)) {
    if (FA_FWD_RESCALE_IN_SLICES) return;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
      for (int j = 0; j < D / 32; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[j][e] *= alpha;
    }
  };

  // acc += P V for the V tile at vb0, with the step's 2 NDMA tile loads
  // (ld: V tile, its first key, K tile, its first key; none if ld[0] < 0)
  // issued one every KP / (2 NDMA) matrix instructions
  constexpr int LD_EVERY = KP / (2 * C::NDMA);
  static_assert(LD_EVERY >= 1 && KP % (2 * C::NDMA) == 0, "load spread");
  // (vpre: the first LA_V V operands, already read by the caller, or null;
  // kout: if not null, the last slices read the first LA_K K operands of the
  // scores at kb_next that follow)
  auto pv = [&](int vb0, const bf16x8_t (&p)[BN / 16], const int (&ld)[4], const bf16x8_t* vpre,
                int kb_next, bf16x8_t* kout) __attribute__((always_inline)) {
    bf16x8_t vr[KP];
#pragma unroll
    for (int k = 0; k < LA_V; ++k) vr[k] = vpre ? vpre[k] : vread(vb0, k);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < KP; ++k) {
      if (k + LA_V < KP) vr[k + LA_V] = vread(vb0, k + LA_V);
      if (kout && k >= KP - LA_K) kout[k - (KP - LA_K)] = kread(kb_next, k - (KP - LA_K));
      if (k % LD_EVERY == LD_EVERY / 2 && ld[0] >= 0) load_part(k / LD_EVERY, ld[0], ld[1], ld[2], ld[3]);
      const int j = k / (BN / 16), kc = k % (BN / 16);
      acc[j] = mfma_32x32x16(vr[k], p[kc], acc[j]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // the step's loads when it has no PV product to carry them
  auto loads_only = [&](const int (&ld)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 2 * C::NDMA; ++j) load_part(j, ld[0], ld[1], ld[2], ld[3]);
  };

  // ---- pipeline over key tiles. K(t) and V(t) live in ring slot t % S.
  // Two schedules share the SIMDs: the workgroup's waves w and w + 4 run on
  // the same SIMD, and the upper half runs its step shifted by half a tile.
  //   lower half, step u: softmax(u) with the scores of tile u+1, rescale,
  //                       then P(u) V(u)                  (vector, then matrix)
  //   upper half, step u: P(u-1) V(u-1), then softmax(u) with the scores of
  //                       tile u+1, rescale               (matrix, then vector)
  // so while one wave of a SIMD runs its exponentials the other feeds the
  // matrix core, and the other way round. Both compute the same thing: acc
  // gains P(t) V(t) before the rescale by alpha(t+1) in either order.
  // Step u reads K(u+1) and V(u) (lower) or V(u-1) (upper), and issues
  // V(u+S-2) and K(u+S): V(u+S-2) replaces V(u-2), last read in step u-1;
  // K(u+S) replaces K(u), last read in step u-1 (every wave passed that
  // step's closing barrier), or for u = 0 by the first tile's scores, which
  // a barrier of their own closes. Loads are issued in the order
  // K0 V0 K1 V1 ... K(S-3) V(S-3) K(S-2) K(S-1), then V(u+S-2) K(u+S) per
  // step, spread over the step's PV product; at the end of step u the next
  // step needs V(u+1) (and the older K(u+2)), after which 2S-5 tiles' loads
  // were issued, so each wave waits until at most that many DMAs are
  // outstanding, then the barrier publishes the tiles to all waves.
  // Operands are read ahead across phase boundaries where their tiles are
  // already published: the lower half reads its first V operands in the
  // last score slices, the upper half its first K operands in the last PV
  // slices and its next step's first V operands (V(u), published since
  // step u began) between its wait and the barrier.
  // Block-sparse: the first keys of the tiles a step loads (u+S-2 for V, u+S
  // for K) and masks (u) come from the list; they are read one step ahead
  // (scalar loads) and passed along, so no step waits for its own list reads.
  // raw list entries of tiles u+S-2, u+S-1, u+S (loads), u (mask) and u-1
  int kw0 = 0, kw1 = 0, kw2 = 0, km = 0, km_prev = 0;
  f32x16_t sA[BN / 32], sB[BN / 32];
  bf16x8_t pA[BN / 16], pB[BN / 16];
  bf16x8_t vpre[LA_V];  // (upper half) V operands read ahead across the barrier


  // Every wave runs every step of the workgroup's key range, with no
  // branch around the work: a tile wholly after a wave's rows (or past N)
  // is masked entirely, which leaves m and l unchanged, gives alpha = 1
  // exactly and P = 0, so acc is unchanged too. A straight path keeps the
  // accumulator in the same registers through the loop. The step count is
  // rounded up to even (the extra step is such a masked tile) so the
  // two-step loop body needs no exit in its middle. Scores of tile u+1 are
  // computed in step u even past the last tile: the ring slot then holds a
  // repeat of the last tile, finite data whose scores go unused.
  //
  // Common head of a step: loads, mask, this step's LDS addresses (through
  // an empty asm statement so the per-chunk XORs are formed here rather than
  // kept live across the loop), row max and alpha.
  auto step_head = [&](int u, f32x16_t (&s_cur)[BN / 32], int& kb0, int& vb0, int v_tile,
                  float& m_use, float& alpha, int (&ld)[4], auto fast) __attribute__((always_inline)) {
    // the step's loads (V tile u+S-2, K tile u+S and their first keys) are
    // issued during its PV product (load_part), not here: right after the
    // barrier every wave would queue its loads at once
    ld[0] = u + S - 2;
    ld[2] = u + S;
    if constexpr (SPARSE) {
      const int nk = list_entry(u + S + 1), nm = list_entry(u + 1);  // for the next step
      ld[1] = entry_key(kw0);
      ld[3] = entry_key(kw2);
      // the even-count padding step (u = n_tiles) is masked entirely
      const int k0 = u < n_tiles ? entry_key(km) : N;
      if (k0 >= N || (CAUSAL && k0 + BN - 1 > row0) || k0 + BN > N) mask(k0, s_cur);
      kw0 = kw1;
      kw1 = kw2;
      kw2 = nk;
      km_prev = km;
      km = nm;
    } else {
      ld[1] = tile_key(u + S - 2);
      ld[3] = tile_key(u + S);
      const int k0 = u * BN;
      if ((CAUSAL && k0 + BN - 1 > row0) || k0 + BN > N) mask(k0, s_cur);
    }
    kb0 = k_addr((u + 1) & (S - 1));
    vb0 = v_addr(v_tile & (S - 1));
    asm volatile("" : "+v"(kb0), "+v"(vb0));
    if constexpr (decltype(fast)::value) {
      // reference fixed for the whole pass (see run below)
      m_use = m_run;
      alpha = 1.f;
      return;
    }
    const float mx = row_max(s_cur);
#if FA_FWD_LAZY_TAU > 0
    // Exactness does not need the true running maximum, only one reference
    // per row used consistently for P, l and acc (and lse at the end); a
    // stale one is kept until a score exceeds it by more than 2^TAU, so P <=
    // 2^TAU and the accumulator rescale is skipped on almost every tile.
    const bool move = __builtin_amdgcn_ballot_w64(mx * c2 > m_run + (float)FA_FWD_LAZY_TAU) != 0;
    const float m_new = move ? fmaxf(m_run, mx * c2) : m_run;
#else
    const float m_new = fmaxf(m_run, mx * c2);
#endif
    m_use = (m_new == -INFINITY) ? 0.f : m_new;
    alpha = exp2_fast(m_run - m_use);
    m_run = m_new;
  };
  // Block-sparse: a tile every key of which follows this wave's last row (or
  // lies past N, as the padding step's does) has P = 0 exactly, and the wave
  // skips its PV product (the scores and softmax stay on the straight path,
  // which keeps the registers where they are). Short lists make such tiles
  // a noticeable share of the work; the dense instances keep the branch-free
  // step, which measured faster there.
  auto dead = [&](int t, int e) {
    if constexpr (SPARSE) {
      const int k0 = t < n_tiles ? entry_key(e) : N;
      return k0 >= N || (CAUSAL && k0 > row0 + 31);
    } else {
      return false;
    }
  };
  // (fast pass: true when a lane's share of a tile's row sum exceeds 2^40
  // or is not finite, i.e. when some P may exceed 2^40.) The test is on the
  // bit pattern: the sum is never negative, so as an unsigned integer every
  // value above 2^40 (0x53800000), +inf and every NaN of either sign lies
  // above that of 2^40. This file is built without NaN semantics, where a
  // float compare may not see a NaN, and the compiler turns some bit tests
  // back into float compares: the empty asm makes the bit pattern an opaque
  // integer, so the test stays an integer compare.
  auto overflow = [&](float lsum) {
    uint32_t bits = __float_as_uint(lsum);
    asm volatile("" : "+v"(bits));
    return __builtin_amdgcn_ballot_w64(bits > 0x53800000u) != 0;
  };
  // (fast pass) A tile whose row sums failed the bound but stayed finite,
  // before its PV: each row's reference moves up by the integer k =
  // floor(log2(row sum over the tile)) + 1 >= 0, and P, the tile's row sum,
  // l and acc are scaled by 2^-k. Scaling by a power of two commutes with the
  // fp32 and bf16 roundings, so the values are exactly those the pass would
  // have formed with the moved reference, and the tile's largest P is now in
  // [2^-7, 1). P's bf16 bit patterns (non-negative) are scaled by a
  // saturating subtraction of k from their exponent fields: a value that
  // would fall below the normal range becomes 0 or a subnormal, 2^-119 or
  // more below the tile's largest P.
  auto rescale_up = [&](bf16x8_t (&p)[BN / 16], float& lsum) __attribute__((always_inline)) {
    const float rt = halves_sum(lsum);
    const int k = max((int)(__float_as_uint(rt) >> 23) - 126, 0);
    m_run += (float)k;
    lsum = __builtin_amdgcn_ldexpf(lsum, -k);
    l_run = __builtin_amdgcn_ldexpf(l_run, -k);
#pragma unroll
    for (int j = 0; j < D / 32; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[j][e] = __builtin_amdgcn_ldexpf(acc[j][e], -k);
    const uint32_t kk = (uint32_t)k << 7;
    const u16x2_t sub = {(uint16_t)kk, (uint16_t)kk};
#pragma unroll
    for (int i = 0; i < BN / 16; ++i) {
      u16x2_t* h = (u16x2_t*)&p[i];
#pragma unroll
      for (int q = 0; q < 4; ++q) h[q] = __builtin_elementwise_sub_sat(h[q], sub);
    }
  };
  // (fast pass) the bookkeeping of a tile whose row sums failed the bound:
  // rescale in place when every sum is finite, else (a score more than 2^128
  // above its reference) flag the wave for the checked pass
  auto on_overflow = [&](bf16x8_t (&p)[BN / 16], float& lsum, bool& bad) __attribute__((always_inline)) {
    uint32_t bits = __float_as_uint(lsum);
    asm volatile("" : "+v"(bits));
    if (__builtin_amdgcn_ballot_w64((bits & 0x7f800000u) == 0x7f800000u)) bad = true;
    else rescale_up(p, lsum);
  };
  auto step_lo = [&](int u, f32x16_t (&s_cur)[BN / 32], f32x16_t (&s_nxt)[BN / 32],
                     bf16x8_t (&p)[BN / 16], auto fast, bool& bad) __attribute__((always_inline)) {
    int kb0, vb0, ld[4];
    float m_use, alpha;
    const bool live = !dead(u, km);
    step_head(u, s_cur, kb0, vb0, u, m_use, alpha, ld, fast);
    bf16x8_t vnext[LA_V];
    float lsum = qk_softmax(kb0, m_use, alpha, s_cur, s_nxt, p, nullptr, vb0, vnext);
    phase_sync();
    if constexpr (decltype(fast)::value) {
      if (overflow(lsum)) on_overflow(p, lsum, bad);
    }
    l_run = l_run * alpha + lsum;
    rescale(alpha);
    if (live) pv(vb0, p, ld, vnext, 0, nullptr);
    else loads_only(ld);
    phase_sync();
    step_sync<C::INFLIGHT>();
  };
  // End of an upper-half step u: like step_sync, but between the wait and
  // the barrier the wave reads the first V operands of step u+1's PV, V(u),
  // so they arrive while it waits for the other waves. V(u) landed before
  // step u began, and its slot is next refilled in step u+2.
  auto step_sync_vpre = [&](int u, bf16x8_t (&vpre)[LA_V]) __attribute__((always_inline)) {
    if constexpr (FA_SAFE_SYNC) asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" :: "n"(C::INFLIGHT) : "memory");
    const int vb_next = v_addr(u & (S - 1));
#pragma unroll
    for (int k = 0; k < LA_V; ++k) vpre[k] = vread(vb_next, k);
    asm volatile("s_barrier" ::: "memory");
  };
  auto step_hi = [&](int u, f32x16_t (&s_cur)[BN / 32], f32x16_t (&s_nxt)[BN / 32],
                     bf16x8_t (&p_cur)[BN / 16], const bf16x8_t (&p_prev)[BN / 16], bool first, auto fast,
                     bool& bad) __attribute__((always_inline)) {
    int kb0, vb0, ld[4];
    float m_use, alpha;
    const bool prev_live = !first && !dead(u - 1, km_prev);
    step_head(u, s_cur, kb0, vb0, u - 1, m_use, alpha, ld, fast);
    bf16x8_t knext[LA_K];
    if (prev_live) {
      pv(vb0, p_prev, ld, vpre, kb0, knext);
    } else {
      loads_only(ld);
#pragma unroll
      for (int i = 0; i < LA_K; ++i) knext[i] = kread(kb0, i);
    }
    phase_sync();
    float lsum = qk_softmax(kb0, m_use, alpha, s_cur, s_nxt, p_cur, knext, 0, nullptr);
    phase_sync();
    if constexpr (decltype(fast)::value) {
      if (overflow(lsum)) on_overflow(p_cur, lsum, bad);
    }
    l_run = l_run * alpha + lsum;
    rescale(alpha);
    step_sync_vpre(u, vpre);
  };

  // One pass over the block's key tiles. Checked pass (fast = false): the
  // lazy reference maximum above, checked on every tile. Fast pass: the
  // reference of every row starts at the maximum of its (masked) scores in
  // the first tile, and no per-tile row maximum is taken. P = 2^(s2 - m_ref)
  // stays exact for any reference; it only needs bounds so that P, l and acc
  // stay in range, and the row sums the softmax forms anyway check them: a
  // lane's share of a tile's row sum above 2^40 makes the wave raise its
  // rows' references by whole powers of two and rescale exactly
  // (rescale_up), after which the pass goes on. No wide underflow can occur:
  // every row's largest P so far is at least 2^-7, so l >= 2^-7. The wave is
  // flagged (returned), and the workgroup runs the block again in the
  // checked pass, when a row sum is not finite (a score more than 2^128
  // above its reference), when a row sees no key of the first tile (a
  // block-sparse list can start with a tile after a row), or when an
  // accumulator is no longer finite at the end (P <= 2^40 bounds l, but acc
  // also scales with |V|).
  auto run = [&](auto fast) __attribute__((always_inline)) {
    m_run = -INFINITY;
    l_run = 0.f;
#pragma unroll
    for (int j = 0; j < D / 32; ++j)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[j][i] = 0.f;
#pragma unroll
    for (int t = 0; t + 2 < S; ++t) {
      const int k0 = tile_key(t);
      load_k(t, k0);
      load_v(t, k0);
    }
    load_k(S - 2, tile_key(S - 2));
    load_k(S - 1, tile_key(S - 1));
    step_sync<C::INFLIGHT>();
    if constexpr (SPARSE) {
      kw0 = list_entry(S - 2);
      kw1 = list_entry(S - 1);
      kw2 = list_entry(S);
      km = list_entry(0);
    }
    qk(k_addr(0), sA);
    // step 0 loads K(S) into slot 0, which every wave has just read: wait
    // until they all have (otherwise only the load's latency keeps a slow
    // wave from reading tile S's keys in place of tile 0's)
    lds_barrier();
    bool bad = false;
    if constexpr (decltype(fast)::value) {
      // (the first tile's key: the mask step_head(0) applies again)
      const int k0 = SPARSE ? entry_key(km) : 0;
      if (k0 + BN > N || (CAUSAL && k0 + BN - 1 > row0)) mask(k0, sA);
      m_run = row_max(sA) * c2;
      // (a row that sees no key of its first tile has no finite reference:
      // the checked pass; an ordered compare, no NaN semantics needed)
      bad = __builtin_amdgcn_ballot_w64(m_run == -INFINITY) != 0;
    }
    const int n_steps = (n_tiles + 1) & ~1;
    if (!FA_FWD_PINGPONG || w < NW / 2) {
      for (int u = 0; u < n_steps; u += 2) {
        step_lo(u, sA, sB, pA, fast, bad);
        step_lo(u + 1, sB, sA, pB, fast, bad);
      }
    } else {
      step_hi(0, sA, sB, pA, pB, true, fast, bad);
      for (int u = 1; u + 1 < n_steps; u += 2) {
        step_hi(u, sB, sA, pB, pA, false, fast, bad);
        step_hi(u + 1, sA, sB, pA, pB, false, fast, bad);
      }
      step_hi(n_steps - 1, sB, sA, pB, pA, false, fast, bad);
      // (the list entries have moved on by one step: km_prev is tile n_steps - 1's)
      const int no_loads[4] = {-1, 0, 0, 0};
      if (!dead(n_steps - 1, km_prev)) pv(v_addr((n_steps - 1) & (S - 1)), pB, no_loads, vpre, 0, nullptr);
    }
    // no load may still be writing this workgroup's LDS when the pass ends
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if constexpr (decltype(fast)::value) {
      // P <= 2^40 bounds l, but acc also scales with |V|: flag the wave if
      // any accumulator value is no longer finite. A sum of the magnitudes
      // is inf or NaN if any term is (additions propagate NaN in every
      // floating-point mode, where a maximum may drop it; a finite sum that
      // overflows only costs a rerun); then the exponent bits of the sum
      // are tested, all ones meaning inf or NaN.
      float asum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < D / 32; ++j)
#pragma unroll
        for (int i = 0; i < 16; ++i) asum[i & 3] += fabsf(acc[j][i]);
      // (opaque integer, as in overflow() above)
      uint32_t bits = __float_as_uint((asum[0] + asum[1]) + (asum[2] + asum[3]));
      asm volatile("" : "+v"(bits));
      bad |= __builtin_amdgcn_ballot_w64((bits & 0x7f800000u) == 0x7f800000u) != 0;
    }
    return bad;
  };
  if constexpr (FAST) {
    // every wave reports, then all rerun together if any was flagged (the
    // passes share barriers); the ring is idle: each wave has waited for its
    // loads, and the barrier below follows every wave's last LDS read
    const bool bad = run(std::true_type{});
    if (bad && lane == 0) redo_flag = 1;
    lds_barrier();
    // (uniform: every lane reads the same word after the barrier)
    if (__builtin_amdgcn_readfirstlane(redo_flag)) run(std::false_type{});
  } else {
    run(std::false_type{});
  }

  // ---- epilogue: O = acc / l, lse = ln(2) * (m + log2 l)
  if (qrow < N) {
    const float l_tot = halves_sum(l_run);
    // (block-sparse rows may see no key at all: O = 0, lse = -inf)
    const float inv = (!SPARSE || l_tot > 0.f) ? 1.f / l_tot : 0.f;
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
    if (h == 0)
      LSE[(size_t)bh * N + qrow] = (!SPARSE || l_tot > 0.f) ? (m_run + log2_fast(l_tot)) * kLn2 : -INFINITY;
  }
}

template <int D, int NW, int BN, int S, bool CAUSAL, bool SPARSE = false>
hipError_t launch(const void* q, const void* k, const void* v, void* o, float* lse,
                  const Problem& p, hipStream_t stream, BlockList sel = BlockList{nullptr, nullptr, 0}) {
  using C = FwdCfg<D, NW, BN, S>;
  const int n_qtiles = (p.N + C::BM - 1) / C::BM;
  const long long grid = (long long)p.B * p.H * n_qtiles;
  const float c2 = p.scale * kLog2e;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, BN, S, CAUSAL, SPARSE>), dim3((unsigned)grid), dim3(C::NT), 0,
                     stream, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)o, lse,
                     p.N, n_qtiles, p.group(), c2, sel.row_ptr, sel.cols, sel.nnz);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                           const Problem& p, hipStream_t stream) {
#ifndef FA_FWD_NW
#define FA_FWD_NW 8
#endif
  static_assert(FwdCfg<128, 8, FA_FWD_BN, FA_FWD_STAGES>::BM == kFwdRowsPerBlock,
                "grid-size limit assumes 256-row blocks");
  if (p.d == 128)
    return p.causal ? launch<128, FA_FWD_NW, FA_FWD_BN, FA_FWD_STAGES, true>(q, k, v, o, lse, p, stream)
                    : launch<128, FA_FWD_NW, FA_FWD_BN, FA_FWD_STAGES, false>(q, k, v, o, lse, p, stream);
  return p.causal ? launch<64, 8, 64, 4, true>(q, k, v, o, lse, p, stream)
                  : launch<64, 8, 64, 4, false>(q, k, v, o, lse, p, stream);
}

hipError_t launch_fwd_bf16_block_sparse(const void* q, const void* k, const void* v, void* o, float* lse,
                                        const int* row_ptr, const int* cols, int nnz, const Problem& p,
                                        hipStream_t stream) {
  // (its own fixed tile shape: the selection is in units of these tiles)
  static_assert(FwdCfg<128, 8, kSparseBlockN, 4>::BM == kSparseBlockM, "block-sparse block shape");
  const BlockList sel{row_ptr, cols, nnz};
  if (p.d == 128)
    return p.causal ? launch<128, 8, kSparseBlockN, 4, true, true>(q, k, v, o, lse, p, stream, sel)
                    : launch<128, 8, kSparseBlockN, 4, false, true>(q, k, v, o, lse, p, stream, sel);
  return p.causal ? launch<64, 8, kSparseBlockN, 4, true, true>(q, k, v, o, lse, p, stream, sel)
                  : launch<64, 8, kSparseBlockN, 4, false, true>(q, k, v, o, lse, p, stream, sel);
}

}  // namespace fa
