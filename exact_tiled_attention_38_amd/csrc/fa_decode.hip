// Decode-shaped attention with the key range split across workgroups, and
// the merge of partial results. bf16 Q/K/V in, fp32 partials, bf16 O and
// fp32 lse out, gfx950.
//
// The method: a few new queries per head (often one) attend to a long cached
// key/value sequence. That is the same exact computation as the forward,
// with almost no reuse of each key byte ("FlashAttention — how 100K-token
// attention fits in memory", section "Arithmetic intensity", contrasts
// decode with prefill), so the kernel is bound by reading K and V once from
// HBM. To put every compute unit on that stream, the keys of each head are
// cut into splits handled by separate workgroups; each split yields a
// partial (O_s, lse_s) per query row, and the splits are combined by the
// rescale identity of online softmax (same page, "Online softmax intuition";
// "Attention and KV Compression", "Tiling and online softmax"):
//     lse = M + ln sum_s e^(lse_s - M),  O = sum_s e^(lse_s - lse) O_s,
// with M = max_s lse_s and empty splits (lse_s = -inf) weighing nothing.
//
// Queries are the last Nq positions of the sequence: with the causal mask,
// query i sees keys j <= Nk - Nq + i. Heads may share keys and values: the
// query heads kvh * group .. + group - 1 read key/value head kvh, and their
// R = group * Nq query rows are contiguous in memory, so one workgroup takes
// all of them (in blocks of 32 rows) and every K/V byte is read once.
//
// Mapping onto CDNA4:
//   * Workgroup = (key/value head, row block of 32 query rows, split) with NW
//     waves. The 32 query rows are the B operand of v_mfma_f32_32x32x16_bf16
//     (rows past R are zero), scores are computed transposed, S^T = K Q^T,
//     and the output accumulates transposed, O^T += V^T P^T, exactly as in
//     the forward: each lane owns one query row and 16 keys of each 32.
//   * The waves of a workgroup take interleaved 32-key tiles of the split.
//     Each wave has its own ring of SLOTS K and V tiles in LDS, filled by
//     non-temporal direct-to-LDS 16-byte loads (each byte is read once, so
//     the caches need not keep it) and refilled as soon as a tile is read, so
//     up to SLOTS - 1 tiles per wave are in flight while it computes; the
//     waves never wait for each other inside the loop.
//   * The mask (keys past the split or past a query's position) is applied
//     to every tile: this kernel is bound by HBM, not by its arithmetic.
//   * At the end the waves' (m, l, acc) merge through LDS by the rescale
//     identity and the split's normalized O_s (fp32) and lse_s go to the
//     workspace; a second kernel merges the splits.
// Scores are kept in log2 units inside the kernel (s2 = s * scale * log2 e).
#include <algorithm>
#include <mutex>

#include "fa.h"
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

static_assert(FA_DECODE_SCRATCH_BYTES == kDecodeScratchBytes, "scratch size of the header and the library");

// Scratch of the no-allocation decode entry point (partial O and lse of the
// key splits, as the caller's workspace holds them otherwise). Every GPU the
// library runs on holds its own copy until the process ends. In host code
// this name is only a stand-in: the device address comes from
// hipGetSymbolAddress, per device, below.
static __device__ __align__(256) char scratch[kDecodeScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Keys per split (about 2 MB of K and V at d = 128) and ring slots per wave.
#ifndef FA_DEC_SPLIT_KEYS
#define FA_DEC_SPLIT_KEYS 4096
#endif
#ifndef FA_DEC_SLOTS128
#define FA_DEC_SLOTS128 2
#endif
// Fewest workgroups a launch is split into: one per compute unit. With the
// non-temporal loads one workgroup's two waves keep enough bytes in flight;
// 320 or 384 leave some compute units with two workgroups and a tail, and
// 512 (two per unit) was 5-6 % slower on the 100K-token and shared-head
// caches (equal on the 16K one)
#ifndef FA_DEC_MIN_WG
#define FA_DEC_MIN_WG 256
#endif
#ifndef FA_DEC_SLOTS64
#define FA_DEC_SLOTS64 4
#endif

constexpr int kDecKeys = 32;  // keys per tile
constexpr int kDecRows = 32;  // query rows per row block

template <int D, int NW, int SLOTS>
struct DecCfg {
  static constexpr int ROWB = 2 * D;              // bytes per K/V row (unpadded)
  static constexpr int TILEB = kDecKeys * ROWB;   // one K (or V) tile
  static constexpr int CPR = D / 8;               // 16-byte chunks per row
  static constexpr int RPW = 1024 / ROWB;         // rows per wave-wide 1 KB load
  static constexpr int NDMA = TILEB / 1024;       // wave-wide loads per tile and tensor
  static constexpr int WAVE_LDS = 2 * SLOTS * TILEB;
  static constexpr int LDS_BYTES = NW * WAVE_LDS;
  // loads issued after the ones of the tile the next step reads
  static constexpr int INFLIGHT = (SLOTS - 1) * 2 * NDMA;
  // wave-merge area: waves 1 .. NW-1 store m, l and D/2 accumulator values per lane
  static constexpr int XFLOATS = D / 2 + 2;
  static_assert((SLOTS & (SLOTS - 1)) == 0 && SLOTS >= 2, "ring slots: power of two");
  static_assert(INFLIGHT <= 63, "vmcnt range");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS capacity");
  static_assert((NW - 1) * 64 * XFLOATS * 4 <= LDS_BYTES, "merge area");
};

template <int N>
__device__ __forceinline__ void wait_loads() {
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}
__device__ __forceinline__ void wait_lds_reads() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// Workspace layout: partial O [S][P][D] fp32, then partial lse [S][P] fp32,
// where P = units * RP padded rows (RP = 32 * row blocks per unit) and the
// padded row of (unit, r) is unit * RP + r.
template <int D, int NW, int SLOTS, bool CAUSAL>
__global__ void __launch_bounds__(64 * NW)
decode_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
              const uint16_t* __restrict__ V, float* __restrict__ Opart, float* __restrict__ Lpart,
              int R, int Nq, int Nk, int n_rblocks, int n_splits, int L, long long P, float c2) {
  using C = DecCfg<D, NW, SLOTS>;
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];
  FA_LDS char* lds = (FA_LDS char*)smem;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, n = lane & 31;

  // workgroup -> (unit, row block, split); the split index runs fastest
  const int bid = blockIdx.x;
  const int rest = __builtin_amdgcn_readfirstlane(bid / n_splits);
  const int s = bid - rest * n_splits;
  const int unit = __builtin_amdgcn_readfirstlane(rest / n_rblocks);
  const int rb = rest - unit * n_rblocks;
  const int k_begin = __builtin_amdgcn_readfirstlane(s * L);
  const int k_last = __builtin_amdgcn_readfirstlane(min(Nk, k_begin + L) - 1);  // last key of the split
  const int span = k_last - k_begin;  // keys in the split, minus one

  // this lane's query row: r = g * Nq + i sits at position Nk - Nq + i
  const int r = rb * kDecRows + n;
  const bool row_ok = r < R;
  const int pos = row_ok ? Nk - Nq + (r % Nq) : Nk - 1;
  // last visible key of this row in the split, relative to k_begin, minus 4h
  const int lim0 = (CAUSAL ? min(pos, k_last) : k_last) - k_begin - 4 * h;

  bf16x8_t qf[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    u32x4_t x = {0u, 0u, 0u, 0u};
    if (row_ok) x = *(const u32x4_t*)(Q + ((size_t)unit * R + r) * D + 16 * c + 8 * h);
    qf[c] = __builtin_bit_cast(bf16x8_t, x);
  }
#pragma unroll
  for (int c = 0; c < D / 16; ++c) asm volatile("" :: "v"(qf[c]));

  const char* Kb = (const char*)(K + ((size_t)unit * Nk + k_begin) * D);
  const char* Vb = (const char*)(V + ((size_t)unit * Nk + k_begin) * D);
  FA_LDS char* kring = lds + w * C::WAVE_LDS;
  FA_LDS char* vring = kring + SLOTS * C::TILEB;

  // this wave's tiles: w, w + NW, w + 2 NW, ... of the split's ceil((span+1)/32)
  const int n_t = span / kDecKeys + 1;
  const int n_w = __builtin_amdgcn_readfirstlane(max(0, (n_t - w + NW - 1) / NW));

  // Step u of this wave loads its tile u into ring slot u % SLOTS. Rows past
  // the split's last key (and whole tiles past the wave's last) are fetched
  // from that last key: in-bounds, finite, and masked or never read.
  const int dma_row = lane / C::CPR, dma_chunk = lane % C::CPR;
  auto load_tile = [&](int u) {
    const int uu = min(u, max(n_w - 1, 0));
    const int k0 = kDecKeys * (w + NW * uu);
    FA_LDS char* kd = kring + (u & (SLOTS - 1)) * C::TILEB;
    FA_LDS char* vd = vring + (u & (SLOTS - 1)) * C::TILEB;
#pragma unroll
    for (int i = 0; i < C::NDMA; ++i) {
      const int row = i * C::RPW + dma_row;
      const uint32_t kr = (uint32_t)min(k0 + row, span) * C::ROWB;
      // (each K/V byte is read once: non-temporal)
      dma16_nt(Kb, kr + 16 * (dma_chunk ^ kswz<D>(row)), kd + i * 1024);
      dma16_nt(Vb, kr + 16 * (dma_chunk ^ vswz<D>(row)), vd + i * 1024);
    }
  };

  // LDS read offsets within a tile, as in the forward: K row n, logical
  // chunk 2c + h at koff0 ^ 32c; transposed V reads at voff0 ^ 64j.
  const int koff0 = n * C::ROWB + 16 * (h ^ kswz<D>(n));
  const int tr_row = 4 * h + ((lane >> 2) & 3);
  const int tr_chunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int voff0 = tr_row * C::ROWB + 16 * (tr_chunk ^ vswz<D>(tr_row)) + 8 * (lane & 1);

  float m_run = -INFINITY, l_run = 0.f;
  f32x16_t acc[D / 32];
#pragma unroll
  for (int j = 0; j < D / 32; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[j][i] = 0.f;

#pragma unroll
  for (int u = 0; u < SLOTS; ++u) load_tile(u);
  wait_loads<C::INFLIGHT>();

  for (int u = 0; u < n_w; ++u) {
    const FA_LDS char* ks = kring + (u & (SLOTS - 1)) * C::TILEB;
    const FA_LDS char* vs = vring + (u & (SLOTS - 1)) * C::TILEB;
    const int k0 = kDecKeys * (w + NW * u);  // first key of the tile, relative to k_begin

    // S^T = K Q^T
    f32x16_t sc = {};
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const bf16x8_t a = *(const FA_LDS bf16x8_t*)(ks + (koff0 ^ (32 * c)));
      sc = mfma_32x32x16(a, qf[c], sc);
    }
    // mask: value i holds key k0 + 8(i/4) + 4h + i%4
    const int lim = lim0 - k0;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (8 * (i >> 2) + (i & 3) > lim) sc[i] = -INFINITY;

    // online softmax update (an all-masked row keeps m = -inf, l = 0, acc = 0)
    float mx = fmaxf(sc[0], sc[1]);
#pragma unroll
    for (int i = 2; i < 16; i += 2) mx = max3(mx, sc[i], sc[i + 1]);
    mx = halves_max(mx);
    const float m_new = fmaxf(m_run, mx * c2);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2_fast(m_run - m_use);
    float lsum = 0.f;
    bf16x8_t pb[2];
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      const float p0 = exp2_fast(fmaf(sc[i], c2, -m_use));
      const float p1 = exp2_fast(fmaf(sc[i + 1], c2, -m_use));
      lsum += p0 + p1;
      const bf16x2_t b = to_bf16x2(p0, p1);
      pb[i >> 3][i & 7] = b[0];
      pb[i >> 3][(i & 7) + 1] = b[1];
    }
    l_run = fmaf(l_run, alpha, lsum);
    m_run = m_new;
#pragma unroll
    for (int j = 0; j < D / 32; ++j)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[j][i] *= alpha;

    // O^T += V^T P^T; the two 16-key steps follow the score registers' key order
#pragma unroll
    for (int j = 0; j < D / 32; ++j)
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        const FA_LDS char* vp = vs + (voff0 ^ (64 * j)) + 16 * kc * C::ROWB;
        const bf16x8_t b = concat8(lds_read_tr4(vp), lds_read_tr4(vp + 8 * C::ROWB));
        acc[j] = mfma_32x32x16(b, pb[kc], acc[j]);
      }

    // slot u is read: refill it with tile u + SLOTS, then wait for tile u + 1
    wait_lds_reads();
    load_tile(u + SLOTS);
    wait_loads<C::INFLIGHT>();
  }
  wait_loads<0>();
  __syncthreads();  // every wave is done with its ring: the LDS becomes the merge area

  FA_LDS float* xs = (FA_LDS float*)smem;  // [NW - 1][XFLOATS][64]
  if (w > 0) {
    FA_LDS float* x = xs + (w - 1) * C::XFLOATS * 64;
    x[lane] = m_run;
    x[64 + lane] = l_run;
#pragma unroll
    for (int j = 0; j < D / 32; ++j)
#pragma unroll
      for (int i = 0; i < 16; ++i) x[(2 + 16 * j + i) * 64 + lane] = acc[j][i];
  }
  __syncthreads();
  if (w != 0) return;

#pragma unroll
  for (int ww = 1; ww < NW; ++ww) {
    const FA_LDS float* x = xs + (ww - 1) * C::XFLOATS * 64;
    const float m2 = x[lane], l2 = x[64 + lane];
    const float m = fmaxf(m_run, m2);
    const float mu = m == -INFINITY ? 0.f : m;
    const float a1 = exp2_fast(m_run - mu), a2 = exp2_fast(m2 - mu);
    l_run = l_run * a1 + l2 * a2;
#pragma unroll
    for (int j = 0; j < D / 32; ++j)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[j][i] = acc[j][i] * a1 + x[(2 + 16 * j + i) * 64 + lane] * a2;
    m_run = m;
  }
  const float l_tot = halves_sum(l_run);
  if (!row_ok) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const long long prow = (long long)unit * (n_rblocks * kDecRows) + r;
  float* orow = Opart + ((size_t)s * P + prow) * D;
#pragma unroll
  for (int j = 0; j < D / 32; ++j)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4_t x = {acc[j][4 * g] * inv, acc[j][4 * g + 1] * inv, acc[j][4 * g + 2] * inv,
                         acc[j][4 * g + 3] * inv};
      *(f32x4_t*)(orow + 32 * j + 8 * g + 4 * h) = x;
    }
  if (h == 0) Lpart[(size_t)s * P + prow] = l_tot > 0.f ? (m_run + log2_fast(l_tot)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------- merge

__device__ __forceinline__ float load_part(const float* p) { return *p; }
__device__ __forceinline__ float load_part(const uint16_t* p) {
  return __uint_as_float((uint32_t)*p << 16);
}

// One wave per output row. Output row o = unit * R + r reads padded row
// unit * RP + r of each of the S parts (part s at Opart + s * P * D). The
// part statistics are spread over the lanes (max and sum by butterfly
// reductions); the weighted sum of the parts runs eight parts at a time so
// their loads overlap.
template <int D, typename Tin>
__global__ void __launch_bounds__(256)
merge_kernel(const Tin* __restrict__ Opart, const float* __restrict__ Lpart, uint16_t* __restrict__ O,
             float* __restrict__ LSE, long long rows, long long R, long long RP, int S, long long P) {
  constexpr int E = D / 64;  // output values per lane
  const long long row = (long long)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const long long unit = row / R;
  const long long prow = unit * RP + (row - unit * R);
  const float* lp = Lpart + prow;
  float m = -INFINITY;
  for (int s = lane; s < S; s += 64) m = fmaxf(m, lp[(size_t)s * P]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  const float mu = m == -INFINITY ? 0.f : m;
  float tot = 0.f;
  for (int s = lane; s < S; s += 64) tot += exp2_fast((lp[(size_t)s * P] - mu) * kLog2e);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) tot += __shfl_xor(tot, o);
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  const Tin* src = Opart + (size_t)prow * D + E * lane;
#pragma unroll 8
  for (int s = 0; s < S; ++s) {
    const float wgt = exp2_fast((lp[(size_t)s * P] - mu) * kLog2e);
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = fmaf(wgt, load_part(src + (size_t)s * P * D + e), acc[e]);
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  uint16_t* dst = O + (size_t)row * D + E * lane;
  if constexpr (E == 2) {
    const bf16x2_t b = to_bf16x2(acc[0] * inv, acc[1] * inv);
    *(uint32_t*)dst = __builtin_bit_cast(uint32_t, b);
  } else {
    const bf16x2_t b = to_bf16x2(acc[0] * inv, 0.f);
    *dst = __builtin_bit_cast(uint16_t, (__bf16)b[0]);
  }
  if (lane == 0) LSE[row] = m == -INFINITY ? -INFINITY : mu + log2_fast(tot) * kLn2;
}

// The same merge for many parts: one workgroup per output row, the parts
// split over its 4 waves (a quarter of the dependent loads each), partial
// sums combined through LDS.
template <int D, typename Tin>
__global__ void __launch_bounds__(256)
merge_wide_kernel(const Tin* __restrict__ Opart, const float* __restrict__ Lpart, uint16_t* __restrict__ O,
                  float* __restrict__ LSE, long long R, long long RP, int S, long long P) {
  constexpr int E = D / 64;
  __shared__ float red[4][D];
  __shared__ float stat[2][4];
  const long long row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const long long unit = row / R;
  const long long prow = unit * RP + (row - unit * R);
  const float* lp = Lpart + prow;
  float m = -INFINITY;
  for (int s = tid; s < S; s += 256) m = fmaxf(m, lp[(size_t)s * P]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if (lane == 0) stat[0][wv] = m;
  __syncthreads();
  m = fmaxf(fmaxf(stat[0][0], stat[0][1]), fmaxf(stat[0][2], stat[0][3]));
  const float mu = m == -INFINITY ? 0.f : m;
  float tot = 0.f;
  for (int s = tid; s < S; s += 256) tot += exp2_fast((lp[(size_t)s * P] - mu) * kLog2e);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) tot += __shfl_xor(tot, o);
  if (lane == 0) stat[1][wv] = tot;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  const Tin* src = Opart + (size_t)prow * D + E * lane;
#pragma unroll 4
  for (int s = wv; s < S; s += 4) {
    const float wgt = exp2_fast((lp[(size_t)s * P] - mu) * kLog2e);
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = fmaf(wgt, load_part(src + (size_t)s * P * D + e), acc[e]);
  }
#pragma unroll
  for (int e = 0; e < E; ++e) red[wv][E * lane + e] = acc[e];
  __syncthreads();
  if (wv != 0) return;
  tot = (stat[1][0] + stat[1][1]) + (stat[1][2] + stat[1][3]);
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e)
    acc[e] = ((red[0][E * lane + e] + red[1][E * lane + e]) + (red[2][E * lane + e] + red[3][E * lane + e])) * inv;
  uint16_t* dst = O + (size_t)row * D + E * lane;
  if constexpr (E == 2) {
    const bf16x2_t b = to_bf16x2(acc[0], acc[1]);
    *(uint32_t*)dst = __builtin_bit_cast(uint32_t, b);
  } else {
    const bf16x2_t b = to_bf16x2(acc[0], 0.f);
    *dst = __builtin_bit_cast(uint16_t, (__bf16)b[0]);
  }
  if (lane == 0) LSE[row] = m == -INFINITY ? -INFINITY : mu + log2_fast(tot) * kLn2;
}

// Parts at or above this count go to the one-workgroup-per-row merge.
constexpr int kWideMergeParts = 16;

template <int D, typename Tin>
hipError_t launch_merge(const Tin* parts, const float* lparts, void* o, float* lse, long long rows,
                        long long R, long long RP, int S, long long P, hipStream_t stream) {
  if (S >= kWideMergeParts) {
    hipLaunchKernelGGL((merge_wide_kernel<D, Tin>), dim3((unsigned)rows), dim3(256), 0, stream, parts, lparts,
                       (uint16_t*)o, lse, R, RP, S, P);
  } else {
    const long long blocks = (rows + 3) / 4;
    hipLaunchKernelGGL((merge_kernel<D, Tin>), dim3((unsigned)blocks), dim3(256), 0, stream, parts, lparts,
                       (uint16_t*)o, lse, rows, R, RP, S, P);
  }
  return hipGetLastError();
}

template <int D, int NW, int SLOTS, bool CAUSAL>
hipError_t launch_decode_t(const void* q, const void* k, const void* v, void* o, float* lse,
                           void* workspace, const DecodeProblem& p, hipStream_t stream) {
  const DecodePlan pl = decode_plan(p);
  float* Opart = (float*)workspace;
  float* Lpart = Opart + (size_t)pl.S * pl.P * p.d;
  const long long grid = (long long)p.B * p.Hkv * pl.n_rblocks * pl.S;
  const float c2 = p.scale * kLog2e;
  hipLaunchKernelGGL((decode_kernel<D, NW, SLOTS, CAUSAL>), dim3((unsigned)grid), dim3(64 * NW), 0, stream,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, Opart, Lpart, pl.R, p.Nq,
                     p.Nk, pl.n_rblocks, pl.S, pl.L, pl.P, c2);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_merge<D, float>(Opart, Lpart, o, lse, (long long)p.B * p.H * p.Nq, pl.R,
                                pl.n_rblocks * kDecRows, pl.S, pl.P, stream);
}

}  // namespace

DecodePlan decode_plan(const DecodeProblem& p) {
  DecodePlan pl;
  const int group = p.H / p.Hkv;
  pl.R = group * p.Nq;
  pl.n_rblocks = (pl.R + kDecRows - 1) / kDecRows;
  pl.P = (long long)p.B * p.Hkv * pl.n_rblocks * kDecRows;
  const long long base = (long long)p.B * p.Hkv * pl.n_rblocks;
  // Splits of about FA_DEC_SPLIT_KEYS keys (long enough that a workgroup's
  // start-up and merge costs are small next to its stream of K and V), but
  // at least FA_DEC_MIN_WG workgroups, and at least 4 tiles per wave.
  const long long tiles = ((long long)p.Nk + kDecKeys - 1) / kDecKeys;
  long long S = std::max(((long long)p.Nk + FA_DEC_SPLIT_KEYS - 1) / FA_DEC_SPLIT_KEYS, (FA_DEC_MIN_WG + base - 1) / base);
  S = std::max(1LL, std::min(S, tiles / (kDecodeWaves * 4)));
  const long long step = (long long)kDecKeys * kDecodeWaves;
  long long L = ((p.Nk + S - 1) / S + step - 1) / step * step;
  pl.L = (int)L;
  pl.S = (int)((p.Nk + L - 1) / L);  // every split non-empty
  return pl;
}

size_t decode_workspace_bytes(const DecodeProblem& p) {
  const DecodePlan pl = decode_plan(p);
  return (size_t)pl.S * pl.P * (p.d + 1) * sizeof(float);
}

hipError_t launch_decode(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace,
                         const DecodeProblem& p, hipStream_t stream) {
  constexpr int NW = kDecodeWaves;
  if (p.d == 128)
    return p.causal ? launch_decode_t<128, NW, FA_DEC_SLOTS128, true>(q, k, v, o, lse, workspace, p, stream)
                    : launch_decode_t<128, NW, FA_DEC_SLOTS128, false>(q, k, v, o, lse, workspace, p, stream);
  return p.causal ? launch_decode_t<64, NW, FA_DEC_SLOTS64, true>(q, k, v, o, lse, workspace, p, stream)
                  : launch_decode_t<64, NW, FA_DEC_SLOTS64, false>(q, k, v, o, lse, workspace, p, stream);
}

hipError_t decode_scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    // once per device, with that device current: its copy's address
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                 const DecodeProblem& p, hipStream_t stream) {
  void* ws = nullptr;
  const hipError_t e = decode_scratch_address(&ws);
  if (e != hipSuccess) return e;
  // (the kernels write every partial before the merge reads it: nothing to clear)
  return launch_decode(q, k, v, o, lse, ws, p, stream);
}

hipError_t launch_merge_bf16(const void* o_parts, const float* lse_parts, void* o, float* lse, int S,
                             long long rows, int d, hipStream_t stream) {
  // one unit holding every row: output row o reads row o of each part
  if (d == 128)
    return launch_merge<128, uint16_t>((const uint16_t*)o_parts, lse_parts, o, lse, rows, rows, rows, S, rows,
                                       stream);
  return launch_merge<64, uint16_t>((const uint16_t*)o_parts, lse_parts, o, lse, rows, rows, rows, S, rows,
                                    stream);
}

}  // namespace fa
