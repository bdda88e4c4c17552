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

// fp8 (e4m3) forward: per-tensor dequantisation factors of Q, K and V.
struct Fp8Scales {
  float q, k, v;
};
hipError_t launch_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, const Problem& p,
                          const Fp8Scales& sc, hipStream_t stream);

// Block-sparse forward: query blocks of kSparseBlockM rows, key blocks of
// kSparseBlockN keys (the forward's own tiles), selection in CSR form.
constexpr int kSparseBlockM = 256;
constexpr int kSparseBlockN = 64;
hipError_t launch_fwd_bf16_block_sparse(const void* q, const void* k, const void* v, void* o, float* lse,
                                        const int* row_ptr, const int* cols, int nnz, const Problem& p,
                                        hipStream_t stream);

// Decode: Nq queries per head at the end of a sequence of Nk keys.
struct DecodeProblem {
  int B, H, Hkv, Nq, Nk, d;
  int causal;
  float scale;
};
// How the decode kernel splits its work (a function of the sizes only).
struct DecodePlan {
  int R;          // query rows per key/value head: (H / Hkv) * Nq
  int n_rblocks;  // blocks of 32 of those rows
  int S;          // key splits
  int L;          // keys per split (the last may hold fewer)
  long long P;    // padded partial rows per split: B * Hkv * n_rblocks * 32
};
#ifndef FA_DEC_WAVES
#define FA_DEC_WAVES 2
#endif
constexpr int kDecodeWaves = FA_DEC_WAVES;
DecodePlan decode_plan(const DecodeProblem& p);
size_t decode_workspace_bytes(const DecodeProblem& p);
hipError_t launch_decode(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace,
                         const DecodeProblem& p, hipStream_t stream);
// Decode with its partials in the library's static per-device scratch
// (kDecodeScratchBytes; the caller checks the size first) instead of a
// caller workspace: no allocation of any kind.
constexpr size_t kDecodeScratchBytes = size_t(32) << 20;
hipError_t launch_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                 const DecodeProblem& p, hipStream_t stream);
// Merge of S bf16 partial outputs [S][rows][d] with their lse [S][rows].
hipError_t launch_merge_bf16(const void* o_parts, const float* lse_parts, void* o, float* lse, int S,
                             long long rows, int d, hipStream_t stream);

}  // namespace fa
