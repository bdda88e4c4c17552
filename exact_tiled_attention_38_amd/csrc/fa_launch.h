// Internal host-side launchers, one per kernel family. Arguments are already
// validated by the C ABI layer (fa_api.hip); each launcher only picks a
// template instance, computes its grid and enqueues it on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa {

struct Problem {
  int B, H, N, d;
  int causal;
  float scale;
  int Hkv;  // key/value heads; query head h reads key/value head h / (H / Hkv)
  int group() const { return H / Hkv; }
};

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                           const Problem& p, hipStream_t stream);

hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                          const Problem& p, hipStream_t stream);

hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const void* o,
                           const void* dO, const float* lse, void* dq, void* dk, void* dv,
                           void* workspace, const Problem& p, hipStream_t stream);

// dQ of the backward by its own kernel (no atomics): Dvec = rowsum(dO * O).
hipError_t launch_bwd_dq(const void* q, const void* k, const void* v, const void* dO,
                         const float* lse, const float* Dvec, void* dq, const Problem& p,
                         hipStream_t stream);

// Query rows per workgroup of the bf16 forward (sets the grid-size limit).
constexpr int kFwdRowsPerBlock = 256;

}  // namespace fa
