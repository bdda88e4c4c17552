// C ABI of libfa.so: argument validation and dispatch to the kernel launchers.
// Every check runs before any HIP call, so invalid arguments never reach the
// device and never initialise the HIP runtime.
#include <cmath>
#include <cstdint>
#include <cstdio>

#include "fa.h"
#include "fa_launch.h"

static_assert(FA_SPARSE_BLOCK_M == fa::kSparseBlockM && FA_SPARSE_BLOCK_N == fa::kSparseBlockN,
              "block-sparse block sizes of the header and the kernels");

namespace {

thread_local char g_launch_error[256] = "kernel launch failed";

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr long double k2p62 = 4.611686018427387904e18L;

// A launch covers fewer than 2^32 work-items in its (one-dimensional) grid.
bool fits_grid(long double blocks, int threads) { return blocks * threads < 4294967296.0L; }

long long ceil_div(long long a, long long b) { return (a + b - 1) / b; }

// Sizes shared by the forward and backward entry points: element counts
// below 2^62 and every kernel grid in range (256-row bf16 forward and dQ
// blocks of 512 threads, 64-row fp32 forward blocks of 64 threads, 128-key
// dK/dV blocks of 256 threads, one thread per 8 values in the backward's row
// preprocessing). Returns FA_OK or the first failing code.
int check_sizes(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  const long double bh = (long double)B * H;
  if (bh * N * d >= k2p62) return FA_ERR_SHAPE;
  if (!fits_grid(bh * ceil_div(N, fa::kFwdRowsPerBlock), 512) || !fits_grid(bh * ceil_div(N, 64), 64) ||
      !fits_grid(bh * ceil_div(N, 128), 256) || !fits_grid(bh * N * (d / 8), 1))
    return FA_ERR_SHAPE;
  return FA_OK;
}

int check_common(int B, int H, int N, int d, int causal, float scale) {
  const int s = check_sizes(B, H, N, d);
  if (s != FA_OK) return s;
  if (causal != 0 && causal != 1) return FA_ERR_UNSUPPORTED;
  if (!(scale > 0.f) || !std::isfinite(scale)) return FA_ERR_SCALE;
  return FA_OK;
}

// Key/value heads: 1 <= Hkv <= H and Hkv divides H.
int check_kv_heads(int H, int Hkv) {
  if (Hkv < 1 || Hkv > H || H % Hkv != 0) return FA_ERR_SHAPE;
  return FA_OK;
}

// Decode sizes: heads as fa_forward_gqa, Nq queries at the end of Nk keys.
int check_decode(int B, int H, int Hkv, int Nq, int Nk, int d, int causal, float scale) {
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (check_kv_heads(H, Hkv) != FA_OK) return FA_ERR_SHAPE;
  if (Nk >= (1 << 24)) return FA_ERR_SHAPE;  // 32-bit byte offsets within a key split
  if ((long double)B * H * Nq * d >= k2p62) return FA_ERR_SHAPE;
  if ((long double)B * Hkv * Nk * d >= k2p62) return FA_ERR_SHAPE;
  // grids: at most ceil(Nk / 64) splits per 32-row query block, up to 256
  // threads per workgroup; the merge takes up to 256 threads per output row
  const long long R = (long long)(H / Hkv) * Nq;
  if (!fits_grid((long double)B * Hkv * ceil_div(R, 32) * ceil_div(Nk, 64), 256)) return FA_ERR_SHAPE;
  if (!fits_grid((long double)B * H * Nq, 256)) return FA_ERR_SHAPE;
  if (causal != 0 && causal != 1) return FA_ERR_UNSUPPORTED;
  if (causal && Nq > Nk) return FA_ERR_SHAPE;
  if (!(scale > 0.f) || !std::isfinite(scale)) return FA_ERR_SCALE;
  return FA_OK;
}

int launch_status(hipError_t e) {
  if (e == hipSuccess) return FA_OK;
  std::snprintf(g_launch_error, sizeof(g_launch_error), "kernel launch failed: %s", hipGetErrorString(e));
  return FA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int fa_forward_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                   int Hkv, int N, int d, int causal, float scale, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  int s = check_common(B, H, N, d, causal, scale);
  if (s == FA_OK) s = check_kv_heads(H, Hkv);
  if (s != FA_OK) return s;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_ALIGN;
  const fa::Problem p{B, H, N, d, causal, scale, Hkv};
  return launch_status(fa::launch_fwd_bf16(q, k, v, o, lse, p, stream));
}

int fa_forward_block_sparse(const void* q, const void* k, const void* v, void* o, float* lse,
                            const int* row_ptr, const int* cols, int nnz, int B, int H, int Hkv, int N, int d,
                            int causal, float scale, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse || !row_ptr || !cols) return FA_ERR_NULL;
  int s = check_common(B, H, N, d, causal, scale);
  if (s == FA_OK) s = check_kv_heads(H, Hkv);
  if (s == FA_OK && nnz < 0) s = FA_ERR_SHAPE;
  if (s != FA_OK) return s;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(row_ptr) & 3u) || (reinterpret_cast<uintptr_t>(cols) & 3u)) return FA_ERR_ALIGN;
  const fa::Problem p{B, H, N, d, causal, scale, Hkv};
  return launch_status(fa::launch_fwd_bf16_block_sparse(q, k, v, o, lse, row_ptr, cols, nnz, p, stream));
}

int fa_forward_fp8(const void* q, const void* k, const void* v, void* o, float* lse, float q_descale,
                   float k_descale, float v_descale, int B, int H, int Hkv, int N, int d, int causal, float scale,
                   hipStream_t stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  int s = check_common(B, H, N, d, causal, scale);
  if (s == FA_OK) s = check_kv_heads(H, Hkv);
  if (s == FA_OK && d != 128) s = FA_ERR_UNSUPPORTED;
  if (s != FA_OK) return s;
  for (float f : {q_descale, k_descale, v_descale})
    if (!(f > 0.f) || !std::isfinite(f)) return FA_ERR_SCALE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_ALIGN;
  const fa::Problem p{B, H, N, d, causal, scale, Hkv};
  return launch_status(fa::launch_fwd_fp8(q, k, v, o, lse, p, fa::Fp8Scales{q_descale, k_descale, v_descale}, stream));
}

int fa_forward(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
               int N, int d, int causal, float scale, hipStream_t stream) {
  return fa_forward_gqa(q, k, v, o, lse, B, H, H, N, d, causal, scale, stream);
}

int fa_forward_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B,
                   int H, int N, int d, int causal, float scale, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  const int s = check_common(B, H, N, d, causal, scale);
  if (s != FA_OK) return s;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_ALIGN;
  const fa::Problem p{B, H, N, d, causal, scale, H};
  return launch_status(fa::launch_fwd_f32(q, k, v, o, lse, p, stream));
}

size_t fa_backward_workspace_bytes(int B, int H, int N, int d) {
  if (check_sizes(B, H, N, d) != FA_OK) return 0;
  return (size_t)B * H * N * 2 * sizeof(float);
}

int fa_backward_gqa(const void* q, const void* k, const void* v, const void* o, const void* dO,
                    const float* lse, void* dq, void* dk, void* dv, void* workspace, int B, int H,
                    int Hkv, int N, int d, int causal, float scale, hipStream_t stream) {
  if (!q || !k || !v || !o || !dO || !lse || !dq || !dk || !dv || !workspace) return FA_ERR_NULL;
  int s = check_common(B, H, N, d, causal, scale);
  if (s == FA_OK) s = check_kv_heads(H, Hkv);
  if (s != FA_OK) return s;
  const void* ptrs[] = {q, k, v, o, dO, lse, dq, dk, dv, workspace};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return FA_ERR_ALIGN;
  const fa::Problem p{B, H, N, d, causal, scale, Hkv};
  return launch_status(fa::launch_bwd_bf16(q, k, v, o, dO, lse, dq, dk, dv, workspace, p, stream));
}

int fa_backward(const void* q, const void* k, const void* v, const void* o, const void* dO,
                const float* lse, void* dq, void* dk, void* dv, void* workspace, int B, int H,
                int N, int d, int causal, float scale, hipStream_t stream) {
  return fa_backward_gqa(q, k, v, o, dO, lse, dq, dk, dv, workspace, B, H, H, N, d, causal, scale,
                         stream);
}

size_t fa_decode_workspace_bytes(int B, int H, int Hkv, int Nq, int Nk, int d) {
  if (check_decode(B, H, Hkv, Nq, Nk, d, 0, 1.f) != FA_OK) return 0;
  return fa::decode_workspace_bytes(fa::DecodeProblem{B, H, Hkv, Nq, Nk, d, 0, 1.f});
}

int fa_decode(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace, int B,
              int H, int Hkv, int Nq, int Nk, int d, int causal, float scale, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse || !workspace) return FA_ERR_NULL;
  const int s = check_decode(B, H, Hkv, Nq, Nk, d, causal, scale);
  if (s != FA_OK) return s;
  const void* ptrs[] = {q, k, v, o, lse, workspace};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return FA_ERR_ALIGN;
  const fa::DecodeProblem p{B, H, Hkv, Nq, Nk, d, causal, scale};
  return launch_status(fa::launch_decode(q, k, v, o, lse, workspace, p, stream));
}

int fa_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv,
                      int Nq, int Nk, int d, int causal, float scale, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  const int s = check_decode(B, H, Hkv, Nq, Nk, d, causal, scale);
  if (s != FA_OK) return s;
  const void* ptrs[] = {q, k, v, o, lse};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return FA_ERR_ALIGN;
  const fa::DecodeProblem p{B, H, Hkv, Nq, Nk, d, causal, scale};
  if (fa::decode_workspace_bytes(p) > fa::kDecodeScratchBytes) return FA_ERR_SCRATCH;
  return launch_status(fa::launch_decode_noalloc(q, k, v, o, lse, p, stream));
}

int fa_merge(const void* o_parts, const float* lse_parts, void* o, float* lse, int S, long long rows,
             int d, hipStream_t stream) {
  if (!o_parts || !lse_parts || !o || !lse) return FA_ERR_NULL;
  if (S < 1 || rows < 1) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if ((long double)S * rows * d >= k2p62 || !fits_grid((long double)rows, 256)) return FA_ERR_SHAPE;
  if (!aligned16(o_parts) || !aligned16(lse_parts) || !aligned16(o) || !aligned16(lse)) return FA_ERR_ALIGN;
  return launch_status(fa::launch_merge_bf16(o_parts, lse_parts, o, lse, S, rows, d, stream));
}

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE:
      return "invalid shape: B, H and N must be >= 1, the key/value heads must divide H, and sizes "
             "within the library's limits";
    case FA_ERR_UNSUPPORTED: return "unsupported argument: d must be 64 or 128 and causal 0 or 1";
    case FA_ERR_ALIGN: return "every pointer must be 16-byte aligned";
    case FA_ERR_SCALE: return "scale must be positive and finite";
    case FA_ERR_LAUNCH: return g_launch_error;
    case FA_ERR_SCRATCH:
      return "the call needs more than the library's static scratch (FA_DECODE_SCRATCH_BYTES; "
             "fa_decode_workspace_bytes gives the need): use fa_decode with a workspace";
    default: return "unknown status";
  }
}

}  // extern "C"
