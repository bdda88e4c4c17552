// Exact tiled attention forward in fp32 end to end (inputs, arithmetic, O).
//
// Same method as the bf16 kernel ("Attention and KV Compression", section
// "Tiling and online softmax"; "FlashAttention — how 100K-token attention fits
// in memory", "Online softmax intuition"), with nothing rounded to bf16, for
// checks that need fp32 accuracy. It is a plain VALU kernel: one wave per
// block of 64 query rows, one query row per lane (q and the output
// accumulator in registers); K/V tiles of 32 keys are staged in LDS and read
// as wave-wide broadcasts, so there are no bank conflicts. Scores are kept in
// log2 units (s2 = s * scale * log2 e) and exponentiated with v_exp_f32.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kF32Rows = 64;  // query rows per workgroup (one wave)
constexpr int kF32Keys = 32;  // keys per K/V tile

template <int D>
__global__ void __launch_bounds__(64)
fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
               float* __restrict__ O, float* __restrict__ LSE, int N, int n_qtiles, int causal,
               float c2) {
  __shared__ __attribute__((aligned(16))) float Ks[kF32Keys][D];
  __shared__ __attribute__((aligned(16))) float Vs[kF32Keys][D];

  const int lane = threadIdx.x;
  const int bh = blockIdx.x / n_qtiles;
  const int t = blockIdx.x - bh * n_qtiles;
  const int q0 = t * kF32Rows;
  const int row = q0 + lane;
  const size_t head = (size_t)bh * N * D;

  float q[D];
#pragma unroll
  for (int c = 0; c < D; c += 4) {
    f32x4_t x = {0.f, 0.f, 0.f, 0.f};
    if (row < N) x = *(const f32x4_t*)(Q + head + (size_t)row * D + c);
    q[c] = x[0]; q[c + 1] = x[1]; q[c + 2] = x[2]; q[c + 3] = x[3];
  }
  float acc[D];
#pragma unroll
  for (int c = 0; c < D; ++c) acc[c] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int kv_end = causal ? min(N, q0 + kF32Rows) : N;
  for (int k0 = 0; k0 < kv_end; k0 += kF32Keys) {
    __syncthreads();  // previous tile fully consumed
    for (int idx = lane * 4; idx < kF32Keys * D; idx += 64 * 4) {
      const int r = idx / D, c = idx % D;
      f32x4_t kx = {0.f, 0.f, 0.f, 0.f}, vx = {0.f, 0.f, 0.f, 0.f};
      if (k0 + r < N) {
        kx = *(const f32x4_t*)(K + head + (size_t)(k0 + r) * D + c);
        vx = *(const f32x4_t*)(V + head + (size_t)(k0 + r) * D + c);
      }
      *(f32x4_t*)&Ks[r][c] = kx;
      *(f32x4_t*)&Vs[r][c] = vx;
    }
    __syncthreads();

    float s[kF32Keys];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kF32Keys; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) dot = fmaf(q[c], Ks[j][c], dot);
      const int key = k0 + j;
      if (key >= N || (causal && key > row)) dot = -INFINITY;
      s[j] = dot;
      mx = fmaxf(mx, dot);
    }
    const float m_new = fmaxf(m_run, mx * c2);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2_fast(m_run - m_use);
    l_run *= alpha;
#pragma unroll
    for (int c = 0; c < D; ++c) acc[c] *= alpha;
#pragma unroll
    for (int j = 0; j < kF32Keys; ++j) {
      const float p = exp2_fast(fmaf(s[j], c2, -m_use));
      l_run += p;
#pragma unroll
      for (int c = 0; c < D; ++c) acc[c] = fmaf(p, Vs[j][c], acc[c]);
    }
    m_run = m_new;
  }

  if (row < N) {
    // true division (not a rounded reciprocal): keeps O exactly 1 when every
    // visible value is 1, and O's error at one rounding
#pragma unroll
    for (int c = 0; c < D; c += 4) {
      f32x4_t x = {acc[c] / l_run, acc[c + 1] / l_run, acc[c + 2] / l_run, acc[c + 3] / l_run};
      *(f32x4_t*)(O + head + (size_t)row * D + c) = x;
    }
    LSE[(size_t)bh * N + row] = (m_run + log2_fast(l_run)) * kLn2;
  }
}

template <int D>
hipError_t launch(const float* q, const float* k, const float* v, float* o, float* lse,
                  const Problem& p, hipStream_t stream) {
  const int n_qtiles = (p.N + kF32Rows - 1) / kF32Rows;
  const long long grid = (long long)p.B * p.H * n_qtiles;
  hipLaunchKernelGGL(fwd_f32_kernel<D>, dim3((unsigned)grid), dim3(64), 0, stream, q, k, v, o, lse,
                     p.N, n_qtiles, p.causal, p.scale * kLog2e);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                          const Problem& p, hipStream_t stream) {
  return p.d == 128 ? launch<128>(q, k, v, o, lse, p, stream) : launch<64>(q, k, v, o, lse, p, stream);
}

}  // namespace fa
