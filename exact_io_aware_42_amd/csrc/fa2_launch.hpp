// Host-side launch interface between the C ABI (fa2_api.cpp) and the kernel translation
// units. Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa2 {

// H counts query heads. K and V have Hkv heads (H a multiple of Hkv; query head h reads K/V head
// h / (H / Hkv)) and kv_bstride elements between batches (Hkv*N*d for their own tensors,
// 2*Hkv*N*d when packed as [B, 2, Hkv, N, d]); dK, dV are written with the same layout.
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, N, d;
  int Hkv;
  long long kv_bstride;
  bool causal;
  float scale_log2;  // |softmax_scale| * log2(e) (log2(e) when the scale is 0)
  uint32_t q_and = ~0u, q_xor = 0u;  // the scale's sign, applied to Q (see OperandSign)
  // dropout on P (dropout false: none): keep iff hash >= drop_thr, kept values scaled by
  // drop_scale; drop_k0/drop_k1 are the keys derived from the seed and offset
  bool dropout = false;
  uint32_t drop_k0 = 0, drop_k1 = 0, drop_thr = 0;
  float drop_scale = 1.f;
  hipStream_t stream;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* delta;  // workspace: -D, D = rowsum(dO * O), fp32 [B, H, N]
  float* lse2;   // workspace: LSE * log2(e), fp32 [B, H, N]
  int B, H, N, d;
  int Hkv;
  long long kv_bstride;
  bool causal;
  float scale;       // softmax_scale (multiplies dQ and dK)
  float scale_log2;  // |softmax_scale| * log2(e) (log2(e) when the scale is 0)
  // the scale's sign (see OperandSign), applied to Q in the dQ kernel and to the resident K
  // rows in the dK/dV kernels
  uint32_t sgn_and = ~0u, sgn_xor = 0u;
  bool dropout = false;  // as in FwdArgs
  uint32_t drop_k0 = 0, drop_k1 = 0, drop_thr = 0;
  float drop_scale = 1.f;
  // with kv_split > 1 the steps of each (key block, K/V head) pair are split over kv_split
  // dK/dV workgroups, which write fp32 partial sums (dK, scaled, then dV, each
  // [kv_split][B*Hkv][N][d]) to kv_part; a reduction adds them in split order
  int kv_split = 1;
  float* kv_part = nullptr;
  hipStream_t stream;
};

// The (query head, query tile) steps of a (key block, K/V head) pair run in one dK/dV
// workgroup unless the pairs alone give fewer workgroups than the target: then each pair's
// steps are cut into `split` equal ranges, the smallest count from 2 to 8 that reaches it (else
// 8), whose partial sums are added afterwards. Targets: 512 workgroups without the causal mask
// (two per CU of a 256-CU part: one round of equal-length workgroups); 1024 with it, whose
// workgroups differ in length (a key block sees the queries after it), so that the longest-
// first order has two rounds to balance (grouped step B4 H16 Hkv4 N2048 d128: split 4 instead
// of 2 measured +9.9% causal; without the mask the larger split measured -4.2%).
constexpr long long kDkdvMinWorkgroups = 512;
constexpr long long kDkdvMinWorkgroupsCausal = 1024;
constexpr int kDkdvMaxSplit = 8;
inline int dkdv_split(int B, int H, int Hkv, int N, int d, bool causal) {
  (void)H;
  // key blocks of the dK/dV kernel without dropout: 64 keys at d = 256, 128 otherwise
  const int bk = d == 256 ? 64 : 128;
  const long long kblocks = (N + bk - 1) / bk;
  const long long base = kblocks * B * Hkv;
  const long long target = causal ? kDkdvMinWorkgroupsCausal : kDkdvMinWorkgroups;
  if (base >= target) return 1;
  for (int s = 2; s < kDkdvMaxSplit; ++s)
    if (base * s >= target) return s;
  return kDkdvMaxSplit;
}
// Heads per window of the causal workgroup order (schedule_tile in fa2_device.hpp): as many
// heads as `budget` bytes of one XCD's L2 hold the streamed tiles of (head_bytes each: K and V
// for the forward and dQ, the query tiles of a K/V head's group for dK/dV), but at least
// enough for the window's blocks to fill the XCD's workgroup slots, and at most the XCD's
// heads (bh_count / 8). budget 0: all of the XCD's heads in one window.
// Budgets: 8 MiB at d = 64 (windows of 16 heads at B8 H32 N2048; 4 MiB, 8 heads, gained
// 2.7% instead of 6.6%); 0 at d >= 128 (see schedule_tile).
#ifndef FA2_WINDOW_BYTES_D64
#define FA2_WINDOW_BYTES_D64 (8ll << 20)
#endif
#ifndef FA2_WINDOW_BYTES_D128
#define FA2_WINDOW_BYTES_D128 0ll
#endif
constexpr int kCusPerXcd = 32;
inline int causal_window(int bh_count, long long head_bytes, int n_blocks, int wg_per_cu,
                         long long budget) {
  const long long hpx = bh_count / 8;
  if (hpx <= 1) return 1;
  if (budget <= 0) return (int)hpx;
  long long w = head_bytes > 0 ? budget / head_bytes : hpx;
  const long long fill = ((long long)kCusPerXcd * wg_per_cu + n_blocks - 1) / n_blocks;
  if (w < fill) w = fill;
  if (w < 1) w = 1;
  if (w > hpx) w = hpx;
  return (int)w;
}
inline long long window_budget(int d) { return d == 64 ? FA2_WINDOW_BYTES_D64 : FA2_WINDOW_BYTES_D128; }

// Size of the backward scratch array that fa2_bwd_noalloc uses in place of a workspace (per
// GPU): room for -D and LSE*log2(e) of up to 2M (batch, head, query) rows.
constexpr size_t kBwdScratchBytes = size_t(16) << 20;

hipError_t launch_fwd(const FwdArgs& a);
hipError_t launch_bwd(const BwdArgs& a);  // dQ (also D and LSE*log2(e)), then dK/dV
hipError_t launch_bwd_pre(const BwdArgs& a);
hipError_t launch_bwd_dkdv(const BwdArgs& a);
hipError_t launch_bwd_dq(const BwdArgs& a);
// launch_bwd with the workspace parts (each part_bytes long) in the library's static scratch
// array of the current device; a.delta, a.lse2 and the split fields are replaced
hipError_t launch_bwd_noalloc(BwdArgs a, size_t part_bytes);

}  // namespace fa2
