/*
 * fa2.h - C ABI of libfa2.so: exact attention forward and backward on one MI355X (gfx950).
 *
 * What is computed
 *   Forward: O = softmax(scale * Q K^T [+ causal mask]) V, row by row, and the per-row
 *   log-sum-exp LSE_i = log sum_j exp(scale * q_i . k_j) over the visible keys j. This is the
 *   standard attention of page "Flash Attention v2", section "Flash Attention v1: Recap /
 *   What v1 Solved", computed with the tiled online softmax of the same page's "Detailed
 *   Algorithm Comparison / Forward Pass Comparison" and the seven steps of page
 *   "flashattention-2", "How FlashAttention-2 Works (Tiled Algorithm)": the N x N score
 *   matrix never reaches device memory. The causal mask keeps keys j <= i (top-left
 *   aligned; queries and keys share the sequence length N); fully masked tiles are skipped
 *   (page "flashattention-2", "FlashAttention-2 Improvements Over v1", causal masking row).
 *   Backward: dQ, dK, dV of that map for a cotangent dO, recomputing the scores block by
 *   block from Q, K and the saved LSE instead of storing P (page "Flash Attention v2",
 *   sections "2. Backward Pass Computation" and "5. Gradient Accumulation"; a separate
 *   backward kernel as on page "FlashAttention-2: Faster Attention with Better Parallelism
 *   and Work Partitioning"). The gradient is the exact softmax gradient:
 *     D_i = sum_c dO_ic O_ic,  dS = P * (dO V^T - D),  dV = P^T dO,
 *     dQ = scale dS K,  dK = scale dS^T Q.
 *
 * Layout and types
 *   q, k, v, o, dout, dq, dk, dv: bfloat16 (raw 16-bit patterns), contiguous row-major
 *   [B, H, N, d] with d fastest. lse: float32 [B, H, N], natural log. All pointers are
 *   device pointers and must be 16-byte aligned. B*H*N*d may exceed 2^31 (64-bit offsets);
 *   one head's slice must stay below 2 GiB (N*d*2 < 2^31 bytes, i.e. N < 8M at d = 128).
 *   Supported head dimensions: d = 64, 128 and 256 (the pages give FlashAttention-2 head
 *   dimensions up to 256: page "Flash Attention v2", "Head Dimension Support"). Any N >= 1
 *   (ragged tails are masked).
 *   Empty problems (B, H or N equal to 0, the others >= 0) are valid: the call checks d and
 *   the scale, does nothing else (pointers are not examined, no HIP call) and returns FA2_OK;
 *   fa2_bwd_workspace_bytes is then 0.
 *
 * Ownership
 *   The caller allocates and owns every buffer. The library never allocates or frees
 *   device memory and keeps no state between calls except a thread-local error code, so
 *   calls are re-entrant and thread-safe. Outputs must not alias inputs or each other.
 *
 * Asynchrony and errors
 *   Arguments are validated on the host before any HIP call. Invalid arguments return
 *   FA2_ERR_INVALID_ARGUMENT (null or misaligned pointers, negative sizes or d <= 0, a
 *   non-finite scale or one whose magnitude times log2(e) overflows a float, i.e. |scale| above
 *   about 2.3e38, a workspace that is too small, sizes beyond the limits above); an
 *   unsupported head dimension returns FA2_ERR_UNSUPPORTED. Otherwise the kernels are enqueued on `stream`
 *   (0 = the default stream) and the call returns FA2_OK, or FA2_ERR_HIP when the launch
 *   fails (the HIP error code is then available from fa2_last_hip_error()). Results are
 *   valid once the stream has been synchronised. No C++ exception crosses this interface.
 */
#ifndef FA2_H_
#define FA2_H_

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa2_status {
  FA2_OK = 0,
  FA2_ERR_INVALID_ARGUMENT = 1,
  FA2_ERR_UNSUPPORTED = 2,
  FA2_ERR_HIP = 3,
  FA2_ERR_SCRATCH_LIMIT = 4  /* fa2_bwd_noalloc: the problem exceeds the static scratch */
} fa2_status;

/* Forward pass. Writes o [B,H,N,d] (bf16) and lse [B,H,N] (fp32).
 * softmax_scale multiplies the scores before the softmax (1/sqrt(d) is the usual choice;
 * page "Flash Attention v2", "Detailed Algorithm Comparison", scores divided by sqrt(d)). Any
 * finite value is valid: 0 weighs the visible keys equally (O_i is the mean of the visible V
 * rows, LSE_i the log of their count), a negative value favours the smallest scores. It
 * enters the kernels as |scale| * log2(e) with the sign carried by the queries (negated, or
 * zeroed for 0). causal != 0 applies the causal mask. Deterministic: identical inputs give
 * identical bits. */
fa2_status fa2_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int N, int d, int causal, float softmax_scale,
                   hipStream_t stream);

/* Bytes of device workspace the backward needs for these sizes: two fp32 [B,H,N] arrays (the
 * row term D = rowsum(dO*O), stored negated as -D, and LSE*log2(e)), each rounded up to 256
 * bytes. Returns 0 for invalid or empty sizes. */
size_t fa2_bwd_workspace_bytes(int B, int H, int N, int d);

/* Backward pass. Inputs: q, k, v, the forward output o and its lse (from fa2_fwd with the
 * same causal flag and scale), and the cotangent dout. Writes dq, dk, dv [B,H,N,d] (bf16,
 * accumulated in fp32). workspace: device buffer of at least fa2_bwd_workspace_bytes(...)
 * bytes, owned by the caller; its contents on entry do not matter and are clobbered. With
 * fa2_bwd_gqa_workspace_bytes(B, H, H, N, d) bytes, small problems split their dK/dV work (see
 * fa2_bwd_gqa). Deterministic (no atomics). Runs fa2_bwd_dq and then the dK/dV stage on
 * `stream`. */
fa2_status fa2_bwd(const void* q, const void* k, const void* v, const void* o,
                   const void* dout, const float* lse, void* dq, void* dk, void* dv,
                   void* workspace, size_t workspace_bytes,
                   int B, int H, int N, int d, int causal, float softmax_scale,
                   hipStream_t stream);

/* The stages of fa2_bwd, for callers that schedule or time them separately (fa2_bwd_dq
 * followed by fa2_bwd_dkdv gives the results of fa2_bwd with a workspace of
 * fa2_bwd_workspace_bytes bytes bit for bit; the stages never split). All take the same
 * workspace.
 *
 * fa2_bwd_dq: dq [B,H,N,d] (bf16) from q, k, v, o, dout and lse. Parallel over blocks of 256
 *   queries at d = 128 (128 at d = 64 and 256); recomputes P and dP block by block, so no
 *   atomics are needed. It also fills the
 *   workspace with -D_i, D_i = sum_c dO_ic O_ic (equal to sum_j P_ij dP_ij, the row term of
 *   the softmax gradient), and LSE_i * log2(e) for fa2_bwd_dkdv. */
fa2_status fa2_bwd_dq(const void* q, const void* k, const void* v, const void* o,
                      const void* dout, const float* lse, void* workspace,
                      size_t workspace_bytes, void* dq, int B, int H, int N, int d, int causal,
                      float softmax_scale, hipStream_t stream);

/* fa2_bwd_dkdv: dk and dv [B,H,N,d] (bf16) from q, k, v, dout and a workspace filled by
 *   fa2_bwd_dq or fa2_bwd_preprocess (earlier on the same stream). Parallel over blocks of 128
 *   keys (64 at d = 256, and with dropout at d = 128); recomputes P block by block. A scale <= 0 reaches this stage through
 *   the resident K rows (negated, or zeroed for 0), dK = scale * dS^T Q as for any scale. */
fa2_status fa2_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout,
                        const void* workspace, size_t workspace_bytes, void* dk, void* dv,
                        int B, int H, int N, int d, int causal, float softmax_scale,
                        hipStream_t stream);

/* fa2_bwd_preprocess: fills the workspace with -D and LSE * log2(e) (the same values
 *   fa2_bwd_dq stores, summed in a different order), for callers that need dK/dV only. */
fa2_status fa2_bwd_preprocess(const void* o, const void* dout, const float* lse,
                              void* workspace, size_t workspace_bytes,
                              int B, int H, int N, int d, hipStream_t stream);

/* Grouped K/V heads and packed K/V (page "Flash Attention v2", "Migration from v1 to v2", names a
 * kvpacked entry point among the v2 functions). q, o, dq: [B, H, N, d]; lse: [B, H, N] as above.
 * k, v and, in the backward, dk, dv: per batch Hkv heads of [N, d], heads contiguous, and
 * kv_batch_stride elements from one batch to the next: Hkv*N*d for tensors of their own, 2*Hkv*N*d
 * for K and V packed as [B, 2, Hkv, N, d] (k = kv, v = kv + Hkv*N*d; the same for dk, dv). H must be
 * a multiple of Hkv; query head h attends to K/V head h / (H / Hkv) (Hkv = 1: one K/V head for
 * all). dK and dV sum the contributions of the query heads of a group in a fixed order
 * (deterministic). kv_batch_stride must be a multiple of 8 and at least Hkv*N*d. Otherwise as
 * fa2_fwd / fa2_bwd (which are these calls with Hkv = H and kv_batch_stride = H*N*d).
 * Small problems: when the (key block of 128 keys, 64 at d = 256; K/V head) pairs are fewer
 * than 512 (1024 under the causal mask) and the workspace holds
 * fa2_bwd_gqa_workspace_bytes(...) bytes, fa2_bwd, fa2_bwd_gqa and fa2_bwd_dropout cut each
 * pair's (query head, query tile) steps into the smallest number of equal ranges, 2..8, that
 * reaches that many workgroups, run by separate dK/dV workgroups, which write fp32 partial sums into the
 * workspace; a last pass adds them in a fixed order (deterministic; the order differs from the
 * unsplit path's, so results may differ from it in the last bits). With only
 * fa2_bwd_workspace_bytes(...) bytes nothing is split. */
fa2_status fa2_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                       int B, int H, int Hkv, int N, int d, long long kv_batch_stride,
                       int causal, float softmax_scale, hipStream_t stream);

/* Workspace bytes that let fa2_bwd (Hkv = H), fa2_bwd_gqa and fa2_bwd_dropout split the dK/dV
 * work of small problems (above): fa2_bwd_workspace_bytes plus, when the causal rule splits into
 * `parts` (the larger of the two rules), 2 * parts * B*Hkv*N*d fp32 partial sums (rounded up to
 * 256 bytes). 0 for invalid or empty sizes or Hkv not dividing H. */
size_t fa2_bwd_gqa_workspace_bytes(int B, int H, int Hkv, int N, int d);

fa2_status fa2_bwd_gqa(const void* q, const void* k, const void* v, const void* o,
                       const void* dout, const float* lse, void* dq, void* dk, void* dv,
                       void* workspace, size_t workspace_bytes, int B, int H, int Hkv, int N,
                       int d, long long kv_batch_stride, int causal, float softmax_scale,
                       hipStream_t stream);

/* Dropout on the attention probabilities (page "Flash Attention v2", "Installation and Usage":
 * flash_attn_func takes dropout_p). Reading: each P[i, j] is kept with probability 1 - p and
 * then scaled by 1 / P(keep), or zeroed, before it multiplies V; the saved lse is that of the
 * undropped softmax. The backward takes the same (dropout_p, seed, offset) and recomputes the
 * same mask:
 *   dV = (P*Z*s)^T dO,  dS = P * (Z*s*(dO V^T) - D),  D_i = sum_c dO_ic O_ic.
 * The mask is a counter-based function of (seed, offset, query head bh = b*H + h, i, j):
 *   h(x)  = the 32-bit PCG-based hash of Jarzynski and Olano (JCGT 9(3), 2020):
 *           s = x*747796405 + 2891336453; w = ((s >> ((s >> 28) + 4)) ^ s) * 277803737;
 *           h = (w >> 22) ^ w                                   (uint32, wrapping)
 *   k0 = h(seed_lo ^ h(seed_hi)), k1 = h(offset_lo ^ h(offset_hi)), a = h(k0 ^ h(k1 ^ bh))
 *   w(i, m) = h(h(a ^ i) ^ m*0x9E3779B9) for the key pair m = j/2 (one word, two keys)
 *   u(i, j) = low 16 bits of w(i, j/2) for even j, high 16 bits for odd j
 *   keep(i, j) = u(i, j) >= t,  t = floor(p * 2^16),  s = 1/(1 - t/2^16)
 * 0 <= dropout_p < 1 (else FA2_ERR_INVALID_ARGUMENT); dropout_p = 0 runs the kernels without
 * dropout (results identical to fa2_fwd_gqa / fa2_bwd_gqa). K/V layout as in the _gqa calls. */
fa2_status fa2_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int Hkv, int N, int d, long long kv_batch_stride,
                           int causal, float softmax_scale, float dropout_p,
                           unsigned long long seed, unsigned long long offset,
                           hipStream_t stream);

fa2_status fa2_bwd_dropout(const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* lse, void* dq, void* dk, void* dv,
                           void* workspace, size_t workspace_bytes, int B, int H, int Hkv,
                           int N, int d, long long kv_batch_stride, int causal,
                           float softmax_scale, float dropout_p, unsigned long long seed,
                           unsigned long long offset, hipStream_t stream);

/* Backward without a workspace argument, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation). Arguments and
 * results as fa2_bwd with a workspace of fa2_bwd_workspace_bytes(B, H, N, d) bytes (the same
 * kernels, so the same bits; no dK/dV split). The workspace is a static array of 16 MiB inside
 * the library, one per GPU, held from the library's load until the process ends; it fits
 * B*H*N <= fa2_bwd_noalloc_max_rows() (2^21) rows, larger problems return
 * FA2_ERR_SCRATCH_LIMIT before any HIP call. The first call on a device looks up that device's
 * copy (hipGetSymbolAddress, no allocation); no call allocates or frees memory. Every call on
 * a GPU shares its copy, so calls that overlap on one GPU (other streams, other threads)
 * race: order them on one stream or serialise them. */
fa2_status fa2_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* lse, void* dq, void* dk, void* dv,
                           int B, int H, int N, int d, int causal, float softmax_scale,
                           hipStream_t stream);

/* The most (batch, head, query) rows fa2_bwd_noalloc accepts: B*H*N up to this value. */
size_t fa2_bwd_noalloc_max_rows(void);

/* Static, human-readable name of a status code. */
const char* fa2_status_string(fa2_status s);

/* HIP error code of the last FA2_ERR_HIP returned on this thread (0 if none). */
int fa2_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FA2_H_ */
