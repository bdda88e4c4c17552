/*
 * fa.h — C ABI of the exact tiled attention library (libfa.so, gfx950 / MI355X).
 *
 * What it computes. Exact dense softmax attention for every (batch b, head h)
 * slice of contiguous [B, H, N, d] tensors:
 *
 *     S = scale * Q K^T          (masked: S[i][j] = -inf for key j > query i when causal)
 *     P = softmax(S) row-wise,   O = P V,   lse[i] = ln sum_j exp(S[i][j])
 *
 * Sources (three web pages, cited by title and section):
 *   "FlashAttention" (tensorlab.fun flagship module), Beat 01 "What problem
 *       existed?": standard attention is score, mask, softmax, weight.
 *   "FlashAttention — how 100K-token attention fits in memory" (llmdaily.org,
 *       day 19): the softmax equation in "But softmax needs the whole row —
 *       right?"; the tile pipeline in "FlashAttention idea"; the rescale in
 *       "Online softmax intuition".
 *   "Attention and KV Compression" (katajob.com), "Tiling and online softmax":
 *       queries are loaded a block at a time, key/value blocks are streamed
 *       past them, each tile's scores live only on chip, a running maximum,
 *       running sum and partial output are rescaled when the maximum rises,
 *       and only the output plus small per-row statistics reach HBM;
 *       "Recomputation in the backward pass": gradients recompute the tiles
 *       from Q, K, V and those statistics instead of storing P.
 *
 * Readings where the pages are silent (the same readings the CPU oracle uses):
 *   - scale is the caller's; the pages' softmax has none. 1/sqrt(d) is usual.
 *   - causal: key j is visible to query i iff j <= i (queries and keys have
 *     the same count N). causal = 0 means no mask.
 *   - the per-row statistic is one fp32 natural-log logsumexp per query row,
 *     in scaled-score units.
 *   - results are exact up to floating-point reassociation; they are not
 *     bitwise equal to any other implementation.
 *
 * Conventions shared by every entry point below:
 *   - Every tensor pointer is a DEVICE pointer (HIP global memory) owned by
 *     the caller. The library never allocates, frees or synchronizes; all work
 *     is enqueued on `stream` (0 = the null stream) and the call returns
 *     before it runs.
 *   - Layout: contiguous row-major [B, H, N, d] (d fastest); lse and the
 *     backward's per-row D are [B, H, N] fp32. bf16 tensors hold raw IEEE
 *     bfloat16 bit patterns (uint16).
 *   - Outputs are fully overwritten and must not alias any input.
 *   - Every pointer must be 16-byte aligned (the kernels use 128-bit loads).
 *   - All argument checks run before any HIP call; a failing check returns
 *     its code and enqueues nothing. A launch failure returns FA_ERR_LAUNCH;
 *     fa_status_string() then includes the HIP error text (per thread).
 *     Faults during execution surface at the caller's next synchronization.
 *   - Supported: B, H, N >= 1; d in {64, 128}; causal in {0, 1};
 *     0 < scale < inf; B*H*N*d < 2^62, and every kernel grid below 2^32
 *     work-items: B*H*ceil(N/256)*512, B*H*ceil(N/64)*64 and B*H*N*d/8
 *     each < 2^32 (at N = 16384, d = 128: B*H < 16384).
 *   - Thread safety: stateless apart from a per-thread error string and,
 *     for fa_decode_noalloc, a lock-guarded per-device address of its
 *     static scratch (whose contents calls on one GPU share).
 *   - Determinism: forward and backward outputs are bitwise reproducible run
 *     to run (no atomics anywhere).
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  FA_OK = 0,
  FA_ERR_NULL = 1,        /* a required pointer is NULL                          */
  FA_ERR_SHAPE = 2,       /* B, H or N < 1, Hkv does not divide H, or a size
                             overflows the limits above                          */
  FA_ERR_UNSUPPORTED = 3, /* d not in {64, 128}, or causal not in {0, 1}          */
  FA_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned                     */
  FA_ERR_SCALE = 5,       /* scale is not positive, or NaN or infinite           */
  FA_ERR_LAUNCH = 6,      /* the HIP kernel launch itself failed                  */
  FA_ERR_SCRATCH = 7      /* fa_decode_noalloc: the call needs more than the
                             static scratch (FA_DECODE_SCRATCH_BYTES)            */
};

/*
 * Forward, bf16 inputs, fp32 accumulation. The tiled online-softmax forward
 * of "Attention and KV Compression", "Tiling and online softmax": for each
 * block of query rows, K/V tiles are streamed through LDS, QK^T and PV run on
 * bf16 matrix cores with fp32 accumulation, and the running max / running sum
 * / output accumulator are rescaled by exp(m_old - m_new) when a tile raises
 * the max ("FlashAttention — how 100K-token attention fits in memory",
 * "Online softmax intuition"). Causal tiles wholly above the diagonal are
 * skipped; ragged tails are predicated.
 *   q, k, v : const bf16 [B, H, N, d]            (inputs)
 *   o       : bf16 [B, H, N, d]                  (output; O rounded to nearest even)
 *   lse     : fp32 [B, H, N]                     (output; natural-log logsumexp)
 * Allocates nothing: no buffer of size O(N^2), or any other, is created.
 */
int fa_forward(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int N, int d, int causal, float scale, hipStream_t stream);

/*
 * Forward with shared key/value heads (grouped-query attention; one key/value
 * head for all query heads is multi-query attention). "Attention and KV
 * Compression", "The composability point": sharing key/value heads changes
 * only how many of them there are, and the tiled forward runs over them
 * unchanged. Query head h of H reads key/value head h / (H / Hkv), so each
 * group of H / Hkv consecutive query heads shares one; per query head the
 * result is exactly fa_forward's on that head's K and V.
 *   q, o : bf16 [B, H, N, d];  k, v : const bf16 [B, Hkv, N, d];  lse : fp32 [B, H, N]
 *   Hkv  : 1 <= Hkv <= H and H % Hkv == 0, else FA_ERR_SHAPE.
 * Everything else as fa_forward, which is this call with Hkv = H.
 */
int fa_forward_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int Hkv, int N, int d, int causal, float scale,
                   hipStream_t stream);

/*
 * Block-sparse forward: attention restricted to selected blocks ("Attention
 * and KV Compression", "The composability point": with sparse selection the
 * tiled kernel runs on the selected blocks only). The (query, key) plane of
 * each head is cut into blocks of FA_SPARSE_BLOCK_M query rows by
 * FA_SPARSE_BLOCK_N keys (the forward's own tiles); query block r of head
 * (b, h), r' = (b * H + h) * ceil(N / FA_SPARSE_BLOCK_M) + r, attends to the
 * key blocks cols[row_ptr[r'] .. row_ptr[r' + 1]). Pairs outside the listed
 * blocks are excluded from the softmax, and with causal = 1 so are keys after
 * the query inside listed blocks. Unselected blocks are never loaded.
 *   q, o         : bf16 [B, H, N, d];  k, v : const bf16 [B, Hkv, N, d]
 *   lse          : fp32 [B, H, N]; a row that sees no key gets O = 0, lse = -inf
 *   row_ptr      : const int32 [B * H * ceil(N / FA_SPARSE_BLOCK_M) + 1], device memory
 *   cols         : const int32 [nnz], device memory; key block indices
 *                  (0 .. ceil(N / FA_SPARSE_BLOCK_N) - 1), any order, no
 *                  repeats within a row (a repeat would count its keys twice)
 * The list is read on the device only: offsets are clamped to [0, nnz] and
 * block indices to their range, so malformed lists give wrong results but
 * never an out-of-bounds access. Heads may be shared as in fa_forward_gqa.
 * row_ptr and cols must be 4-byte aligned; other rules as fa_forward.
 */
#define FA_SPARSE_BLOCK_M 256
#define FA_SPARSE_BLOCK_N 64
int fa_forward_block_sparse(const void* q, const void* k, const void* v, void* o, float* lse,
                            const int* row_ptr, const int* cols, int nnz, int B, int H, int Hkv, int N,
                            int d, int causal, float scale, hipStream_t stream);

/*
 * Forward on fp8 inputs: the narrower number format that "Attention and KV
 * Compression", "What it does and does not change", names as a later
 * refinement. Q, K, V hold OCP e4m3 codes (1 sign, 4 exponent bits with bias
 * 7, 3 mantissa bits; largest finite 448) with one fp32 dequantisation factor
 * per tensor: the attention computed is the exact one of code * factor. Both
 * products run on the fp8 matrix cores with fp32 accumulation; P is rounded
 * to e4m3 before the PV product (the only rounding beyond fp32), O is bf16.
 *   q    : const e4m3 [B, H, N, d];  k, v : const e4m3 [B, Hkv, N, d]
 *   o    : bf16 [B, H, N, d];  lse : fp32 [B, H, N] (of the dequantised scores)
 *   q_descale, k_descale, v_descale : finite and > 0, else FA_ERR_SCALE
 * d must be 128 (else FA_ERR_UNSUPPORTED); other rules as fa_forward_gqa.
 */
int fa_forward_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                   float q_descale, float k_descale, float v_descale, int B, int H, int Hkv, int N,
                   int d, int causal, float scale, hipStream_t stream);

/*
 * Forward, fp32 inputs, fp32 arithmetic, fp32 output: the same tiled
 * computation ("Attention and KV Compression", "Tiling and online softmax":
 * query blocks, streamed key/value tiles, running maximum, sum and partial
 * output rescaled as the maximum rises, only O and the per-row statistic
 * written; the rescale as in "FlashAttention — how 100K-token attention fits
 * in memory", "Online softmax intuition"), without bf16 rounding anywhere,
 * for checks that need fp32 accuracy. Same arguments as fa_forward, all
 * tensors fp32.
 */
int fa_forward_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                   int B, int H, int N, int d, int causal, float scale, hipStream_t stream);

/*
 * Bytes of device workspace fa_backward needs: the fp32 per-row
 * D = rowsum(dO * O) [B, H, N] followed by the fp32 per-row lse * log2(e)
 * [B, H, N], i.e. B*H*N*8 bytes, O(N). Returns 0 for invalid sizes.
 */
size_t fa_backward_workspace_bytes(int B, int H, int N, int d);

/*
 * Backward with recomputation ("Attention and KV Compression", "Recomputation
 * in the backward pass"; "FlashAttention — how 100K-token attention fits in
 * memory", "Training backward"). P is never stored: each (query tile, key
 * tile) pair recomputes S = scale Q K^T and P = exp(S - lse) from the saved
 * lse, then
 *     dV += P^T dO,  dP = dO V^T,  D = rowsum(dO * O),  dS = P * (dP - D),
 *     dK += scale dS^T Q,  dQ += scale dS K.
 * Three kernels run on `stream`: D, then dK/dV (one workgroup per key block
 * streaming the query tiles), then dQ (one workgroup per query block
 * streaming the key tiles; S and dP are recomputed there too). No atomics:
 * dq, dk and dv are bitwise reproducible.
 *   q, k, v, o, dO : const bf16 [B, H, N, d]  (o and lse as fa_forward wrote them)
 *   lse            : const fp32 [B, H, N]
 *   dq, dk, dv     : bf16 [B, H, N, d]        (outputs)
 *   workspace      : device scratch of fa_backward_workspace_bytes(B, H, N, d)
 *                    bytes, 16-byte aligned; its contents on entry do not
 *                    matter (the library writes what it reads).
 * Two calls may not share a workspace concurrently.
 */
int fa_backward(const void* q, const void* k, const void* v, const void* o, const void* dO,
                const float* lse, void* dq, void* dk, void* dv, void* workspace,
                int B, int H, int N, int d, int causal, float scale, hipStream_t stream);

/*
 * Backward of fa_forward_gqa. The gradient of a shared key/value head is the
 * sum of what each query head of its group sends it (the chain rule over a
 * shared input); the dK/dV kernel streams the query tiles of all heads of the
 * group through one key block and sums them in registers, so dk and dv are
 * written once, with no atomics, and stay bitwise reproducible.
 *   q, o, dO, dq : bf16 [B, H, N, d];  k, v, dk, dv : bf16 [B, Hkv, N, d];
 *   lse : const fp32 [B, H, N];  Hkv as fa_forward_gqa;
 *   workspace : fa_backward_workspace_bytes(B, H, N, d) bytes (per query head).
 * Everything else as fa_backward, which is this call with Hkv = H.
 */
int fa_backward_gqa(const void* q, const void* k, const void* v, const void* o, const void* dO,
                    const float* lse, void* dq, void* dk, void* dv, void* workspace,
                    int B, int H, int Hkv, int N, int d, int causal, float scale,
                    hipStream_t stream);

/*
 * Decode: Nq new queries per head (typically 1, or a few) against a cached
 * sequence of Nk keys, the workload that "FlashAttention — how 100K-token
 * attention fits in memory", "Arithmetic intensity", sets against prefill:
 * the same exact attention, bound by reading K and V once. The queries are
 * the last Nq positions of the sequence; with causal = 1 query i sees keys
 * j <= Nk - Nq + i (with Nq = 1 every key; Nq = Nk is fa_forward's mask).
 * Key/value heads may be shared as in fa_forward_gqa.
 * The keys of each head are split across workgroups; each split writes a
 * partial (O_s, lse_s) into the workspace and a second kernel merges them
 * by the rescale identity of online softmax ("Online softmax intuition";
 * "Attention and KV Compression", "Tiling and online softmax"), as fa_merge
 * does.
 *   q, o      : bf16 [B, H, Nq, d];  k, v : const bf16 [B, Hkv, Nk, d] (the cache)
 *   lse       : fp32 [B, H, Nq] (output, natural log)
 *   workspace : fa_decode_workspace_bytes(...) bytes of device memory,
 *               16-byte aligned; contents on entry do not matter.
 * Limits: Nk < 2^24; B*Hkv*ceil(H/Hkv*Nq/32)*ceil(Nk/64)*256 < 2^32 and
 * B*H*Nq*256 < 2^32; causal requires Nq <= Nk (else FA_ERR_SHAPE). The
 * split count is a function of the sizes only, so results are bitwise
 * reproducible. Two calls may not share a workspace concurrently.
 */
size_t fa_decode_workspace_bytes(int B, int H, int Hkv, int Nq, int Nk, int d);
int fa_decode(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace,
              int B, int H, int Hkv, int Nq, int Nk, int d, int causal, float scale,
              hipStream_t stream);

/*
 * fa_decode for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, and harnesses that forbid allocation.
 * Same arguments as fa_decode without the workspace, same kernels and the
 * same results bit for bit; the split partials live instead in one static
 * scratch array of FA_DECODE_SCRATCH_BYTES inside the library, of which
 * every GPU the library runs on holds its own copy until the process ends.
 * The call allocates and frees nothing (its first call on a device looks up
 * that device's copy of the array, with the device current).
 *   Sizes whose fa_decode_workspace_bytes exceeds FA_DECODE_SCRATCH_BYTES
 *   return FA_ERR_SCRATCH before any HIP call; other checks as fa_decode.
 *   All calls on one GPU share its scratch: calls that may overlap on one
 *   GPU (other streams, other threads) race and give wrong results; calls
 *   ordered on one stream are safe, each overwriting the last one's partials.
 */
#define FA_DECODE_SCRATCH_BYTES (32u << 20)
int fa_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int H, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                      hipStream_t stream);

/*
 * Merge S partial attention results computed over disjoint sets of keys
 * into the result over their union ("Online softmax intuition": the rescale
 * that lets blockwise processing reach the exact softmax), for example the
 * outputs of fa_forward on key shards (non-causal) held by different
 * devices:
 *     M = max_s lse_s,  lse = M + ln sum_s e^(lse_s - M),
 *     o = sum_s e^(lse_s - lse) o_s.
 * A part with lse_s = -inf (no visible key) weighs nothing; a row whose
 * parts are all -inf gets o = 0 and lse = -inf.
 *   o_parts   : const bf16 [S, rows, d]  (part s is a [rows, d] block)
 *   lse_parts : const fp32 [S, rows]     (natural log, as fa_forward writes it)
 *   o         : bf16 [rows, d];  lse : fp32 [rows]  (outputs)
 * S >= 1, 1 <= rows < 2^24, S*rows*d < 2^62, d in {64, 128}.
 */
int fa_merge(const void* o_parts, const float* lse_parts, void* o, float* lse, int S,
             long long rows, int d, hipStream_t stream);

/* Static text for a status code; for FA_ERR_LAUNCH the text of the calling
 * thread's last HIP launch error. Never NULL. */
const char* fa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
