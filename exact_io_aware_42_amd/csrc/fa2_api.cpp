// C ABI of libfa2.so (declared in include/fa2.h): host-side validation, then the kernel
// launches on the caller's stream. No device memory is allocated here.
#include "fa2.h"

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <initializer_list>

#include "fa2_launch.hpp"

namespace {

thread_local int g_last_hip_error = 0;

constexpr double kLog2e = 1.4426950408889634074;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shared size checks. Returns FA2_OK or the status to report; *empty is set when B, H or N is 0
// (a valid call with nothing to compute).
// Head dimensions 64, 128 and 256.
fa2_status check_sizes(int B, int H, int N, int d, float scale, bool* empty, int max_d = 256) {
  *empty = false;
  if (B < 0 || H < 0 || N < 0 || d <= 0) return FA2_ERR_INVALID_ARGUMENT;
  // any finite scale whose magnitude times log2(e) is a finite float
  if (!std::isfinite(scale) || !std::isfinite(static_cast<float>(std::fabs(scale) * kLog2e)))
    return FA2_ERR_INVALID_ARGUMENT;
  if ((d != 64 && d != 128 && d != 256) || d > max_d) return FA2_ERR_UNSUPPORTED;
  if (B == 0 || H == 0 || N == 0) {
    *empty = true;
    return FA2_OK;
  }
  const unsigned long long elems =
      (unsigned long long)B * (unsigned long long)H * (unsigned long long)N * (unsigned long long)d;
  if (elems > (1ull << 46)) return FA2_ERR_INVALID_ARGUMENT;
  // one head's Q/K/V slice is addressed with 32-bit buffer offsets
  if ((unsigned long long)N * (unsigned long long)d * 2ull >= (1ull << 31))
    return FA2_ERR_INVALID_ARGUMENT;
  // the workgroup grid (B*H*ceil(N/64)) must fit a 32-bit dimension
  if ((unsigned long long)B * H * ((unsigned long long)(N + 63) / 64) > 0x7fffffffull)
    return FA2_ERR_INVALID_ARGUMENT;
  return FA2_OK;
}

// How the kernels apply a softmax scale of any sign (they need a positive multiplier c): c =
// |scale| * log2(e) with one operand of the score product negated when the scale is negative,
// or zeroed (every score 0) with c = log2(e) when it is 0. Masks for the operand's bf16 pairs:
// x -> (x & and_mask) ^ xor_mask.
struct ScaleForm {
  float scale_log2;
  uint32_t and_mask, xor_mask;
};
ScaleForm scale_form(float scale) {
  ScaleForm f;
  f.and_mask = scale == 0.0f ? 0u : ~0u;
  f.xor_mask = scale < 0.0f ? 0x80008000u : 0u;
  f.scale_log2 =
      scale == 0.0f ? static_cast<float>(kLog2e) : static_cast<float>(std::fabs(scale) * kLog2e);
  return f;
}

fa2_status from_hip(hipError_t e) {
  if (e == hipSuccess) return FA2_OK;
  g_last_hip_error = static_cast<int>(e);
  return FA2_ERR_HIP;
}

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

// Dropout keys and threshold (the mask generator is documented in fa2.h): the same 32-bit hash
// the kernels use, applied on the host to the seed and offset halves.
uint32_t host_pcg_hash(uint32_t x) {
  const uint32_t state = x * 747796405u + 2891336453u;
  const uint32_t word = ((state >> ((state >> 28u) + 4u)) ^ state) * 277803737u;
  return (word >> 22u) ^ word;
}

struct DropHost {
  uint32_t k0, k1, thr;
  float scale;
};

// FA2_OK and the parameters for 0 < p < 1; p outside [0, 1) is invalid.
fa2_status drop_params(float p, unsigned long long seed, unsigned long long offset,
                       DropHost* out) {
  if (!(p >= 0.0f && p < 1.0f)) return FA2_ERR_INVALID_ARGUMENT;
  const double t = std::min(std::floor((double)p * 65536.0), 65535.0);  // 16-bit uniforms
  out->thr = (uint32_t)t << 16;
  out->scale = (float)(65536.0 / (65536.0 - t));
  out->k0 = host_pcg_hash((uint32_t)seed ^ host_pcg_hash((uint32_t)(seed >> 32)));
  out->k1 = host_pcg_hash((uint32_t)offset ^ host_pcg_hash((uint32_t)(offset >> 32)));
  return FA2_OK;
}

// K/V head count and batch stride (elements) for grouped or packed K/V. FA2_OK or the status.
fa2_status check_kv(int B, int H, int Hkv, int N, int d, long long kv_bstride) {
  if (Hkv <= 0 || H % Hkv != 0) return FA2_ERR_INVALID_ARGUMENT;
  const long long head = (long long)N * d;
  if (kv_bstride < (long long)Hkv * head || (kv_bstride & 7) != 0) return FA2_ERR_INVALID_ARGUMENT;
  // the grid of the dK/dV kernels and the K/V extent
  if ((unsigned long long)B * Hkv * ((unsigned long long)(N + 63) / 64) > 0x7fffffffull)
    return FA2_ERR_INVALID_ARGUMENT;
  if ((unsigned long long)kv_bstride > (1ull << 50)) return FA2_ERR_INVALID_ARGUMENT;
  return FA2_OK;
}

fa2_status fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                    int H, int Hkv, int N, int d, long long kv_bstride, int causal,
                    float softmax_scale, hipStream_t stream, float dropout_p = 0.f,
                    unsigned long long seed = 0, unsigned long long offset = 0) {
  bool empty;
  fa2_status st = check_sizes(B, H, N, d, softmax_scale, &empty);
  if (st != FA2_OK) return st;
  DropHost drop;
  st = drop_params(dropout_p, seed, offset, &drop);
  if (st != FA2_OK || empty) return st;
  st = check_kv(B, H, Hkv, N, d, kv_bstride);
  if (st != FA2_OK) return st;
  const void* ptrs[] = {q, k, v, o, lse};
  for (const void* p : ptrs)
    if (p == nullptr || !aligned16(p)) return FA2_ERR_INVALID_ARGUMENT;
  fa2::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.B = B;
  a.H = H;
  a.N = N;
  a.d = d;
  a.Hkv = Hkv;
  a.kv_bstride = kv_bstride;
  a.causal = causal != 0;
  const ScaleForm sf = scale_form(softmax_scale);
  a.scale_log2 = sf.scale_log2;
  a.q_and = sf.and_mask;
  a.q_xor = sf.xor_mask;
  a.dropout = dropout_p > 0.f;
  a.drop_k0 = drop.k0;
  a.drop_k1 = drop.k1;
  a.drop_thr = drop.thr;
  a.drop_scale = drop.scale;
  a.stream = stream;
  return from_hip(fa2::launch_fwd(a));
}

}  // namespace

extern "C" {

fa2_status fa2_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                   int H, int N, int d, int causal, float softmax_scale, hipStream_t stream) {
  return fwd_impl(q, k, v, o, lse, B, H, H, N, d, (long long)H * N * d, causal, softmax_scale,
                  stream);
}

fa2_status fa2_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                       int H, int Hkv, int N, int d, long long kv_batch_stride, int causal,
                       float softmax_scale, hipStream_t stream) {
  return fwd_impl(q, k, v, o, lse, B, H, Hkv, N, d, kv_batch_stride, causal, softmax_scale,
                  stream);
}

fa2_status fa2_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int Hkv, int N, int d, long long kv_batch_stride,
                           int causal, float softmax_scale, float dropout_p,
                           unsigned long long seed, unsigned long long offset,
                           hipStream_t stream) {
  return fwd_impl(q, k, v, o, lse, B, H, Hkv, N, d, kv_batch_stride, causal, softmax_scale,
                  stream, dropout_p, seed, offset);
}

// Workspace layout: -D, D = rowsum(dO * O) [B*H*N floats], then LSE * log2(e) [B*H*N floats],
// the second part starting at a 256-byte boundary.
static size_t ws_part_bytes(int B, int H, int N) { return round256((size_t)B * H * N * sizeof(float)); }

size_t fa2_bwd_workspace_bytes(int B, int H, int N, int d) {
  bool empty;
  if (check_sizes(B, H, N, d, 1.0f, &empty) != FA2_OK || empty) return 0;
  return 2 * ws_part_bytes(B, H, N);
}

size_t fa2_bwd_gqa_workspace_bytes(int B, int H, int Hkv, int N, int d) {
  bool empty;
  if (check_sizes(B, H, N, d, 1.0f, &empty) != FA2_OK || empty) return 0;
  if (Hkv <= 0 || H % Hkv != 0) return 0;
  // sized for the causal split, the larger of the two
  const int split = fa2::dkdv_split(B, H, Hkv, N, d, true);
  const size_t part = split > 1 ? round256((size_t)2 * split * B * Hkv * N * d * sizeof(float)) : 0;
  return 2 * ws_part_bytes(B, H, N) + part;
}

namespace {

// Split the dK/dV work of each (key block, K/V head) pair when the problem is too small to fill
// the chip and the workspace holds the partial sums (fa2_bwd_gqa_workspace_bytes); with the
// smaller workspace nothing is split.
void set_kv_split(fa2::BwdArgs* a, void* workspace, size_t workspace_bytes) {
  const int split = fa2::dkdv_split(a->B, a->H, a->Hkv, a->N, a->d, a->causal);
  if (split > 1 &&
      workspace_bytes >= fa2_bwd_gqa_workspace_bytes(a->B, a->H, a->Hkv, a->N, a->d)) {
    a->kv_split = split;
    a->kv_part = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                          2 * ws_part_bytes(a->B, a->H, a->N));
  }
}

// The backward argument block without its workspace fields (sizes already validated).
void fill_bwd_args(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                   int causal, float softmax_scale, hipStream_t stream, fa2::BwdArgs* a) {
  a->q = q;
  a->k = k;
  a->v = v;
  a->o = o;
  a->dout = dout;
  a->lse = lse;
  a->dq = dq;
  a->dk = dk;
  a->dv = dv;
  a->B = B;
  a->H = H;
  a->N = N;
  a->d = d;
  a->Hkv = H;
  a->kv_bstride = (long long)H * N * d;
  a->causal = causal != 0;
  a->scale = softmax_scale;
  const ScaleForm sf = scale_form(softmax_scale);
  a->scale_log2 = sf.scale_log2;
  a->sgn_and = sf.and_mask;
  a->sgn_xor = sf.xor_mask;
  a->stream = stream;
}

fa2_status bwd_args(const void* q, const void* k, const void* v, const void* o, const void* dout,
                    const float* lse, void* workspace, size_t workspace_bytes, void* dq, void* dk,
                    void* dv, int B, int H, int N, int d, int causal, float softmax_scale,
                    hipStream_t stream, fa2::BwdArgs* a, bool* empty) {
  const fa2_status st = check_sizes(B, H, N, d, softmax_scale, empty);
  if (st != FA2_OK || *empty) return st;
  if (workspace == nullptr || !aligned16(workspace) ||
      workspace_bytes < fa2_bwd_workspace_bytes(B, H, N, d))
    return FA2_ERR_INVALID_ARGUMENT;
  fill_bwd_args(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, causal, softmax_scale, stream, a);
  a->delta = static_cast<float*>(workspace);
  a->lse2 = reinterpret_cast<float*>(static_cast<char*>(workspace) + ws_part_bytes(B, H, N));
  return FA2_OK;
}

bool all_ok(std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs)
    if (p == nullptr || !aligned16(p)) return false;
  return true;
}

}  // namespace

fa2_status fa2_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, void* dq, void* dk, void* dv, void* workspace,
                   size_t workspace_bytes, int B, int H, int N, int d, int causal,
                   float softmax_scale, hipStream_t stream) {
  fa2::BwdArgs a;
  bool empty;
  const fa2_status st = bwd_args(q, k, v, o, dout, lse, workspace, workspace_bytes, dq, dk, dv,
                                 B, H, N, d, causal, softmax_scale, stream, &a, &empty);
  if (st != FA2_OK || empty) return st;
  if (!all_ok({q, k, v, o, dout, lse, dq, dk, dv})) return FA2_ERR_INVALID_ARGUMENT;
  set_kv_split(&a, workspace, workspace_bytes);
  return from_hip(fa2::launch_bwd(a));
}

fa2_status fa2_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* lse, void* dq, void* dk, void* dv,
                           int B, int H, int N, int d, int causal, float softmax_scale,
                           hipStream_t stream) {
  bool empty;
  const fa2_status st = check_sizes(B, H, N, d, softmax_scale, &empty);
  if (st != FA2_OK || empty) return st;
  if (!all_ok({q, k, v, o, dout, lse, dq, dk, dv})) return FA2_ERR_INVALID_ARGUMENT;
  const size_t part = ws_part_bytes(B, H, N);
  if (2 * part > fa2::kBwdScratchBytes) return FA2_ERR_SCRATCH_LIMIT;
  // fa2_bwd's arguments; the workspace parts come from the static scratch array
  fa2::BwdArgs a;
  fill_bwd_args(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, causal, softmax_scale, stream, &a);
  return from_hip(fa2::launch_bwd_noalloc(a, part));
}

size_t fa2_bwd_noalloc_max_rows(void) { return fa2::kBwdScratchBytes / (2 * sizeof(float)); }

fa2_status fa2_bwd_gqa(const void* q, const void* k, const void* v, const void* o,
                       const void* dout, const float* lse, void* dq, void* dk, void* dv,
                       void* workspace, size_t workspace_bytes, int B, int H, int Hkv, int N,
                       int d, long long kv_batch_stride, int causal, float softmax_scale,
                       hipStream_t stream) {
  fa2::BwdArgs a;
  bool empty;
  fa2_status st = bwd_args(q, k, v, o, dout, lse, workspace, workspace_bytes, dq, dk, dv, B, H,
                           N, d, causal, softmax_scale, stream, &a, &empty);
  if (st != FA2_OK || empty) return st;
  st = check_kv(B, H, Hkv, N, d, kv_batch_stride);
  if (st != FA2_OK) return st;
  if (!all_ok({q, k, v, o, dout, lse, dq, dk, dv})) return FA2_ERR_INVALID_ARGUMENT;
  a.Hkv = Hkv;
  a.kv_bstride = kv_batch_stride;
  set_kv_split(&a, workspace, workspace_bytes);
  return from_hip(fa2::launch_bwd(a));
}

fa2_status fa2_bwd_dropout(const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* lse, void* dq, void* dk, void* dv,
                           void* workspace, size_t workspace_bytes, int B, int H, int Hkv,
                           int N, int d, long long kv_batch_stride, int causal,
                           float softmax_scale, float dropout_p, unsigned long long seed,
                           unsigned long long offset, hipStream_t stream) {
  fa2::BwdArgs a;
  bool empty;
  fa2_status st = bwd_args(q, k, v, o, dout, lse, workspace, workspace_bytes, dq, dk, dv, B, H,
                           N, d, causal, softmax_scale, stream, &a, &empty);
  if (st != FA2_OK) return st;
  DropHost drop;
  st = drop_params(dropout_p, seed, offset, &drop);
  if (st != FA2_OK || empty) return st;
  st = check_kv(B, H, Hkv, N, d, kv_batch_stride);
  if (st != FA2_OK) return st;
  if (!all_ok({q, k, v, o, dout, lse, dq, dk, dv})) return FA2_ERR_INVALID_ARGUMENT;
  a.Hkv = Hkv;
  a.kv_bstride = kv_batch_stride;
  a.dropout = dropout_p > 0.f;
  a.drop_k0 = drop.k0;
  a.drop_k1 = drop.k1;
  a.drop_thr = drop.thr;
  a.drop_scale = drop.scale;
  set_kv_split(&a, workspace, workspace_bytes);
  return from_hip(fa2::launch_bwd(a));
}

fa2_status fa2_bwd_preprocess(const void* o, const void* dout, const float* lse, void* workspace,
                              size_t workspace_bytes, int B, int H, int N, int d,
                              hipStream_t stream) {
  fa2::BwdArgs a;
  bool empty;
  const fa2_status st = bwd_args(nullptr, nullptr, nullptr, o, dout, lse, workspace,
                                 workspace_bytes, nullptr, nullptr, nullptr, B, H, N, d, 0, 1.0f,
                                 stream, &a, &empty);
  if (st != FA2_OK || empty) return st;
  if (!all_ok({o, dout, lse})) return FA2_ERR_INVALID_ARGUMENT;
  return from_hip(fa2::launch_bwd_pre(a));
}

fa2_status fa2_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout,
                        const void* workspace, size_t workspace_bytes, void* dk, void* dv, int B,
                        int H, int N, int d, int causal, float softmax_scale, hipStream_t stream) {
  fa2::BwdArgs a;
  bool empty;
  const fa2_status st = bwd_args(q, k, v, nullptr, dout, nullptr, const_cast<void*>(workspace),
                                 workspace_bytes, nullptr, dk, dv, B, H, N, d, causal,
                                 softmax_scale, stream, &a, &empty);
  if (st != FA2_OK || empty) return st;
  if (!all_ok({q, k, v, dout, dk, dv})) return FA2_ERR_INVALID_ARGUMENT;
  return from_hip(fa2::launch_bwd_dkdv(a));
}

fa2_status fa2_bwd_dq(const void* q, const void* k, const void* v, const void* o,
                      const void* dout, const float* lse, void* workspace,
                      size_t workspace_bytes, void* dq, int B, int H, int N, int d, int causal,
                      float softmax_scale, hipStream_t stream) {
  fa2::BwdArgs a;
  bool empty;
  const fa2_status st = bwd_args(q, k, v, o, dout, lse, workspace, workspace_bytes, dq, nullptr,
                                 nullptr, B, H, N, d, causal, softmax_scale, stream, &a, &empty);
  if (st != FA2_OK || empty) return st;
  if (!all_ok({q, k, v, o, dout, lse, dq})) return FA2_ERR_INVALID_ARGUMENT;
  return from_hip(fa2::launch_bwd_dq(a));
}

const char* fa2_status_string(fa2_status s) {
  switch (s) {
    case FA2_OK:
      return "FA2_OK";
    case FA2_ERR_INVALID_ARGUMENT:
      return "FA2_ERR_INVALID_ARGUMENT";
    case FA2_ERR_UNSUPPORTED:
      return "FA2_ERR_UNSUPPORTED";
    case FA2_ERR_HIP:
      return "FA2_ERR_HIP";
    case FA2_ERR_SCRATCH_LIMIT:
      return "FA2_ERR_SCRATCH_LIMIT";
  }
  return "FA2_UNKNOWN_STATUS";
}

int fa2_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
