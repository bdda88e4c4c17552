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
//   1. preprocess: D_i = sum_k dO_ik O_ik (fp32) and zero the fp32 dQ accumulator.
//   2. dkdv: one workgroup per block of 128 keys of one head, 4 waves x 32 keys.
//      K and V rows of the wave stay in registers (the B operands of S = Q K^T
//      and dP = dO V^T); the fp32 dK^T and dV^T accumulators stay in registers
//      for the whole key block. Query tiles of 64 rows stream through LDS
//      (Q, dO, lse, D). In this orientation each lane owns one key and 16 of
//      every 32 queries, so P and dS feed the dV^T = dO^T P and dK^T = Q^T dS
//      products straight from registers, with dO^T and Q^T read from the
//      row-major LDS tiles by ds_read_b64_tr_b16. dS^T (bf16) is staged in LDS
//      and the workgroup then forms its 64 x d slice of dS K (the keys are the
//      contraction) and adds it to the fp32 dQ accumulator with atomics.
//      Causal: query tiles that end before the key block starts are never
//      visited; waves whose keys all follow the tile's last query skip it.
//   3. dq_convert: dQ accumulator -> bf16 dq.
// dk and dv are deterministic; dq is not (atomic accumulation order).
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kBwdWaves = 4;
constexpr int kBwdKeys = 32 * kBwdWaves;  // keys per workgroup
constexpr int kBwdRows = 64;              // query rows per tile

// LDS pitches (bf16 elements). Q/dO tiles are read both row-wise (128-bit) and
// transposed (ds_read_b64_tr_b16); D + 40 keeps the 16-row 128-bit reads
// conflict-free and limits the transposed reads to 2-way. K and dS^T are only
// read transposed: a row pitch of 16 banks mod 64 spreads each read's 4 rows
// over distinct banks.
template <int D> struct BwdCfg {
  static constexpr int QP = D + 40;
  static constexpr int KP = D + 32;
  static constexpr int SP = kBwdRows + 32;
};

// ---------------------------------------------------------------- preprocess

template <int D>
__global__ void __launch_bounds__(256)
bwd_preprocess_kernel(const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO,
                      float* __restrict__ Dvec, float* __restrict__ dQacc, long long rows) {
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
    const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
    *(f32x4_t*)(dQacc + off) = z;
    *(f32x4_t*)(dQacc + off + 4) = z;
  }
#pragma unroll
  for (int x = LPR / 2; x >= 1; x >>= 1) sum += __shfl_xor(sum, x, LPR);
  if (row < rows && sub == 0) Dvec[row] = sum;
}

// ---------------------------------------------------------------- dq convert

__global__ void __launch_bounds__(256)
bwd_dq_convert_kernel(const float* __restrict__ dQacc, uint16_t* __restrict__ dq, long long n8) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  const f32x4_t a = *(const f32x4_t*)(dQacc + 8 * i);
  const f32x4_t b = *(const f32x4_t*)(dQacc + 8 * i + 4);
  const bf16x2_t p0 = to_bf16x2(a[0], a[1]), p1 = to_bf16x2(a[2], a[3]);
  const bf16x2_t p2 = to_bf16x2(b[0], b[1]), p3 = to_bf16x2(b[2], b[3]);
  u32x4_t out = {__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                 __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3)};
  *(u32x4_t*)(dq + 8 * i) = out;
}

// ---------------------------------------------------------------- dK / dV (+ dQ)

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(64 * kBwdWaves, 1)
bwd_dkdv_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                const float* __restrict__ LSE, const float* __restrict__ Dvec,
                float* __restrict__ dQacc, uint16_t* __restrict__ dK, uint16_t* __restrict__ dV,
                int N, int n_kblocks, float c2, float scale) {
  using C = BwdCfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t Qs[kBwdRows * C::QP];
  __shared__ __attribute__((aligned(16))) uint16_t dOs[kBwdRows * C::QP];
  __shared__ __attribute__((aligned(16))) uint16_t Kt[kBwdKeys * C::KP];
  __shared__ __attribute__((aligned(16))) uint16_t dSt[kBwdKeys * C::SP];
  __shared__ __attribute__((aligned(16))) float lse2s[kBwdRows];
  __shared__ __attribute__((aligned(16))) float Ds[kBwdRows];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, n = lane & 31;
  const int bh = blockIdx.x / n_kblocks;
  const int kbi = blockIdx.x - bh * n_kblocks;
  const int kb0 = kbi * kBwdKeys;
  const int kw0 = kb0 + 32 * w;
  const int key = kw0 + n;
  const size_t head = (size_t)bh * N * D;
  const uint16_t* Qh = Q + head;
  const uint16_t* dOh = dO + head;

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
  // the workgroup's K block, row-major in LDS (for the dQ product)
  for (int ch = tid; ch < kBwdKeys * D / 8; ch += 64 * kBwdWaves) {
    const int r = ch / (D / 8), cc = ch % (D / 8);
    u32x4_t x = {0u, 0u, 0u, 0u};
    if (kb0 + r < N) x = *(const u32x4_t*)(K + head + (size_t)(kb0 + r) * D + cc * 8);
    *(u32x4_t*)(Kt + r * C::KP + cc * 8) = x;
  }

  f32x16_t dvacc[D / 32], dkacc[D / 32];
#pragma unroll
  for (int j = 0; j < D / 32; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) { dvacc[j][i] = 0.f; dkacc[j][i] = 0.f; }

  const int tr_row = 4 * h + ((lane >> 2) & 3);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int n_qtiles = (N + kBwdRows - 1) / kBwdRows;
  const int t_first = CAUSAL ? kb0 / kBwdRows : 0;

  for (int t = t_first; t < n_qtiles; ++t) {
    const int q0 = t * kBwdRows;
    __syncthreads();  // previous tile's readers of Qs/dOs/dSt are done
    for (int ch = tid; ch < kBwdRows * D / 8; ch += 64 * kBwdWaves) {
      const int r = ch / (D / 8), cc = ch % (D / 8);
      u32x4_t a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
      if (q0 + r < N) {
        a = *(const u32x4_t*)(Qh + (size_t)(q0 + r) * D + cc * 8);
        b = *(const u32x4_t*)(dOh + (size_t)(q0 + r) * D + cc * 8);
      }
      *(u32x4_t*)(Qs + r * C::QP + cc * 8) = a;
      *(u32x4_t*)(dOs + r * C::QP + cc * 8) = b;
    }
    if (tid < kBwdRows) {
      const int q = q0 + tid;
      // rows past N get lse = +inf, hence P = 0 and dS = 0
      lse2s[tid] = q < N ? LSE[(size_t)bh * N + q] * kLog2e : INFINITY;
      Ds[tid] = q < N ? Dvec[(size_t)bh * N + q] : 0.f;
    }
    __syncthreads();

    const bool active = !CAUSAL || (kw0 <= q0 + kBwdRows - 1);
    if (active) {
#pragma unroll
      for (int qb = 0; qb < kBwdRows / 32; ++qb) {
        // S = Q K^T and dP = dO V^T for 32 queries x this wave's 32 keys;
        // lane holds key `key`, queries qb*32 + 8(i/4) + 4h + i%4
        f32x16_t s, dp;
#pragma unroll
        for (int i = 0; i < 16; ++i) { s[i] = 0.f; dp[i] = 0.f; }
#pragma unroll
        for (int c = 0; c < D / 16; ++c) {
          const bf16x8_t qa = *(const bf16x8_t*)(Qs + (qb * 32 + n) * C::QP + 16 * c + 8 * h);
          const bf16x8_t ga = *(const bf16x8_t*)(dOs + (qb * 32 + n) * C::QP + 16 * c + 8 * h);
          s = mfma_32x32x16(qa, kf[c], s);
          dp = mfma_32x32x16(ga, vf[c], dp);
        }
        bf16x8_t pb[2], dsb[2];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int qi = qb * 32 + 8 * g + 4 * h;
          const f32x4_t l4 = *(const f32x4_t*)(lse2s + qi);
          const f32x4_t d4 = *(const f32x4_t*)(Ds + qi);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 4 * g + e;
            float p = exp2_fast(fmaf(s[i], c2, -l4[e]));
            if ((CAUSAL && key > q0 + qi + e) || key >= N) p = 0.f;
            const float ds = p * (dp[i] - d4[e]);
            pb[i >> 3][i & 7] = (__bf16)p;
            dsb[i >> 3][i & 7] = (__bf16)ds;
          }
        }
        // dV^T += dO^T P and dK^T += Q^T dS (queries are the contraction)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const int r = qb * 32 + 16 * jj + tr_row;
#pragma unroll
          for (int j = 0; j < D / 32; ++j) {
            const uint16_t* gp = dOs + r * C::QP + 32 * j + tr_col;
            const uint16_t* qp = Qs + r * C::QP + 32 * j + tr_col;
            const bf16x8_t ga = concat8(lds_read_tr4(gp), lds_read_tr4(gp + 8 * C::QP));
            const bf16x8_t qa = concat8(lds_read_tr4(qp), lds_read_tr4(qp + 8 * C::QP));
            dvacc[j] = mfma_32x32x16(ga, pb[jj], dvacc[j]);
            dkacc[j] = mfma_32x32x16(qa, dsb[jj], dkacc[j]);
          }
        }
        // dS^T -> LDS: row = this key, 4 consecutive queries per store
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int i = 4 * g;
          const bf16x4_t v4 = {dsb[i >> 3][i & 7], dsb[i >> 3][(i & 7) + 1], dsb[i >> 3][(i & 7) + 2],
                               dsb[i >> 3][(i & 7) + 3]};
          *(bf16x4_t*)(dSt + (32 * w + n) * C::SP + qb * 32 + 8 * g + 4 * h) = v4;
        }
      }
    } else {
      const u32x2_t z = {0u, 0u};
#pragma unroll
      for (int qb = 0; qb < kBwdRows / 32; ++qb)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *(u32x2_t*)(dSt + (32 * w + n) * C::SP + qb * 32 + 8 * g + 4 * h) = z;
    }
    __syncthreads();

    // dQ[q0 .. q0+63][:] += scale * dS K over this workgroup's 128 keys.
    // (query block, d block) pairs are spread over the waves.
    constexpr int PAIRS = (kBwdRows / 32) * (D / 32);
    for (int pr = w; pr < PAIRS; pr += kBwdWaves) {
      const int qb = pr / (D / 32), j = pr % (D / 32);
      f32x16_t acc;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
      for (int kc = 0; kc < kBwdKeys / 16; ++kc) {
        const int r = 16 * kc + 8 * h + ((lane >> 2) & 3);
        const uint16_t* sp = dSt + r * C::SP + qb * 32 + tr_col;
        const uint16_t* kp = Kt + r * C::KP + 32 * j + tr_col;
        const bf16x8_t a = concat8(lds_read_tr4(sp), lds_read_tr4(sp + 4 * C::SP));
        const bf16x8_t b = concat8(lds_read_tr4(kp), lds_read_tr4(kp + 4 * C::KP));
        acc = mfma_32x32x16(a, b, acc);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int q = q0 + qb * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
        if (q < N) atomicAdd(dQacc + head + (size_t)q * D + 32 * j + n, scale * acc[i]);
      }
    }
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
  float* dQacc = (float*)workspace;
  float* Dvec = dQacc + rows * D;
  {
    const long long threads = rows * (D / 8);
    const long long blocks = (threads + 255) / 256;
    hipLaunchKernelGGL(bwd_preprocess_kernel<D>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const uint16_t*)o, (const uint16_t*)dO, Dvec, dQacc, rows);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    const int n_kblocks = (p.N + kBwdKeys - 1) / kBwdKeys;
    const long long blocks = (long long)p.B * p.H * n_kblocks;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3((unsigned)blocks), dim3(64 * kBwdWaves), 0,
                       stream, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                       (const uint16_t*)dO, lse, (const float*)Dvec, dQacc, (uint16_t*)dk,
                       (uint16_t*)dv, p.N, n_kblocks, p.scale * kLog2e, p.scale);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    const long long n8 = rows * D / 8;
    const long long blocks = (n8 + 255) / 256;
    hipLaunchKernelGGL(bwd_dq_convert_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const float*)dQacc, (uint16_t*)dq, n8);
  }
  return hipGetLastError();
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
