// FlashAttention-2 forward for gfx950: O = softmax(scale Q K^T [+ causal]) V and LSE.
//
// Follows the tiled online-softmax forward (page "Flash Attention v2", "Detailed Algorithm
// Comparison / Forward Pass Comparison"; page "flashattention-2", "How FlashAttention-2
// Works (Tiled Algorithm)") with the three FlashAttention-2 changes (page "FlashAttention-2
// paper", section "Three changes"): the grid also splits the query dimension, so one head
// fills the chip; each wavefront owns 32 query rows and keeps their accumulator, running
// max and running sums in registers; the rescale by exp(m_old - m_new) is deferred until a
// tile's exponentials could exceed 2^8 (no per-tile max is taken until then) and the 1/l
// normalisation happens once at the end. Fully masked causal tiles are skipped (page
// "flashattention-2", "FlashAttention-2 Improvements Over v1").
//
// gfx950 mapping (one workgroup = 8 waves = 256 query rows at d >= 128, 4 waves = 128 rows at
// d = 64; key tiles of 64):
//  * scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: lane l owns
//    query l%32 of its wave, so row max and row sums are in-lane plus one exchange with lane
//    l^32; Q^T fragments (the B operand) stay in VGPRs for the whole key loop;
//  * O^T = V^T P^T with the same MFMA: P^T is the B operand straight from the score
//    registers (the kmap key order makes the layouts agree), V^T fragments come from the
//    row-major V tile through the transposing LDS read, and each lane's O^T column is its own
//    query, so the rescale and the final 1/l are per-lane scalars;
//  * K and V tiles move HBM -> LDS by buffer loads that write LDS directly (no VGPR staging,
//    zero fill past the sequence end), into row-major tiles whose 16-byte chunks are XOR-
//    swizzled so both LDS read patterns are free of bank conflicts, in a ring of four K and
//    four V tiles at d >= 128 (two at d = 64): tiles are taken in groups of two (one at d = 64),
//    the next group streams in while one is computed, and the workgroup meets at one barrier
//    per group;
//  * exp2 form: p = exp2(s * scale*log2(e) - m) is one FMA + one v_exp_f32. Masked tiles
//    (causal diagonal, ragged tail) start their score accumulators at -inf instead of 0 for
//    hidden keys. Two waves per SIMD (three at d = 64) let one wave's softmax VALU work
//    overlap another wave's MFMAs. The key loop is unrolled over the ring so the LDS slot of
//    a tile is a compile-time constant and every LDS address is a base register plus an
//    immediate;
//  * the LSE uses the fp32 sum of the unrounded p. O is normalised by the sum of the weights
//    the PV MFMA actually used: on masked tiles (causal diagonal, ragged tail) a correction
//    sum(bf16(p)) - sum(p) is added, so a row whose visible keys all lie in masked tiles (every
//    causal row with fewer than 64 keys, where O mixes only a few V rows) gets exactly
//    convex bf16 weights; on unmasked tiles the fp32 sum stands in (rows with >= 64 keys, where
//    the difference averages out);
//  * the O tile leaves through LDS (after the last tile's barrier) as whole row segments;
//  * head dimension 256: key tiles of 32 (the O^T and Q^T registers leave room for one MFMA
//    key block of scores);
//  * dropout (DROP): each kept p is multiplied by 1 (and the 1/P(keep) scale joins 1/l at the
//    end), each dropped p by 0, before the PV MFMA; the sums for l and the LSE are those of the
//    undropped p. The keep bits come from the counter-based hash in fa2_device.hpp, one hash
//    word per key pair.
#include <type_traits>

#include "fa2_device.hpp"
#include "fa2_launch.hpp"

namespace fa2 {

namespace {

#ifndef FA2_FWD_OCC
#define FA2_FWD_OCC 2  // waves per SIMD the forward kernel is compiled for
#endif
// Key tiles per workgroup barrier at d >= 128. The 8 waves of a workgroup drift apart within a
// tile (two per SIMD take turns), and a per-wave timer probe put 12-15% of their time at the
// per-tile barrier, also in the long non-causal forward; two tiles per barrier (a ring of 4+4
// tiles, 128 KiB) measured +0.6-1.4% at d = 128 and +1.6-1.8% at d = 256 on every forward
// workload.
#ifndef FA2_FWD_TILES_PER_SYNC
#define FA2_FWD_TILES_PER_SYNC 2
#endif

constexpr float kRescaleSum = 256.0f;  // a lane's partial sum of p per tile stays <= 2^8
constexpr float kRescaleLog2 = 8.0f;   // so each p stays <= 2^8 (log2 units)

// Key tiles of 64 for d <= 128; of 32 at d = 256, where O^T (128 registers) and the resident
// Q^T fragments (64) leave room for one 32-key score block only. A K or V tile is 16 KiB
// (8 KiB at d = 64) either way.
// Workgroup = NW waves of 32 query rows sharing each K/V tile: 8 waves (256 rows, one workgroup
// per CU) for d >= 128, which halves the L2 -> LDS tile traffic per FLOP of 4 waves (+1-3.5%);
// 4 waves at d = 64, whose ~140 registers let three workgroups share a CU (3 waves per SIMD;
// 8-wave workgroups would leave 2 and ran 7-10% slower).
template <int D>
struct FwdShape {
  static constexpr int NW = D == 64 ? 4 : 8;     // waves per workgroup
  static constexpr int BR = 32 * NW;             // query rows per workgroup
  static constexpr int THREADS = 64 * NW;
  static constexpr int BC = D == 256 ? 32 : 64;  // keys per tile
  static constexpr int KB = BC / 32;             // 32-key MFMA blocks per tile
  static constexpr int DCH = D / 8;            // 16-byte chunks per K/V row
  static constexpr int KK = D / 16;            // MFMA k-steps of the score GEMM
  static constexpr int CB = D / 32;            // 32-row blocks of O^T
  static constexpr int TILE_BYTES = BC * D * 2;
  static constexpr int LOADS = TILE_BYTES / (THREADS * 16);  // 16-byte loads per lane per tile
  // tiles per barrier: the LDS ring holds 2*TPB K tiles and as many V tiles (128 KiB at d >= 128,
  // one workgroup per CU); d = 64 keeps 1 so that three workgroups fit a CU
  static constexpr int TPB = D == 64 ? 1 : FA2_FWD_TILES_PER_SYNC;
  static constexpr int SLOTS = 2 * TPB;
  static constexpr int K_SLOT0 = 0;
  static constexpr int V_SLOT0 = SLOTS * TILE_BYTES;
  static constexpr int RING = 2 * SLOTS * TILE_BYTES;
  static constexpr int SMEM =
      RING > NW * store_scratch_bytes(CB) ? RING : NW * store_scratch_bytes(CB);
  static_assert(LOADS >= 1 && DCH >= 8, "tile shape");
  static_assert(TPB == 1 || TPB == 2, "tiles per barrier");
  // every LDS read is a base register plus a 16-bit immediate: the slot offsets within the K
  // and within the V region stay below 64 KiB (the V region's base is in the registers)
  static_assert(SLOTS * TILE_BYTES <= 65536, "ring immediates");
};

template <int D, bool CAUSAL, bool DROP>
__global__ __launch_bounds__(FwdShape<D>::THREADS, FA2_FWD_OCC) void fa2_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ o, float* __restrict__ lse,
    int N, int n_qblocks, int bh_count, int window, int n_qheads, int group,
    long long kv_bstride, float scale_log2, OperandSign qsign, DropParams drop) {
  using S = FwdShape<D>;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[S::SMEM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int g = lane >> 5;

  const TileCoord tc = schedule_tile<CAUSAL ? Order::kLongDescending : Order::kHeadMajor>(
      blockIdx.x, n_qblocks, bh_count, window);
  const size_t head_off = (size_t)tc.bh * (size_t)N * D;
  // K/V head of this query head (grouped heads share one; batch stride may be packed)
  const int b_idx = tc.bh / n_qheads;
  const size_t kv_off = (size_t)b_idx * (size_t)kv_bstride +
                        (size_t)((tc.bh - b_idx * n_qheads) / group) * (size_t)N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(q + head_off, head_bytes);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + kv_off, head_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(v + kv_off, head_bytes);

  const int q_block0 = tc.qb * S::BR;
  const int q_wave0 = q_block0 + wave * 32;
  const int my_q = q_wave0 + l32;
  // dropout: the row key of this lane's query (unused without dropout)
  const uint32_t drop_row =
      DROP ? pcg_hash(drop_head_key(drop, (uint32_t)tc.bh) ^ (uint32_t)my_q) : 0u;

  // ---- key tiles this workgroup visits, and the last one not fully masked for this wave
  constexpr int BC = S::BC;
  int n_tiles = (N + BC - 1) / BC;
  if (CAUSAL) n_tiles = min(N - 1, q_block0 + S::BR - 1) / BC + 1;
  const int wave_last = CAUSAL ? min(n_tiles - 1, (q_wave0 + 31) / BC) : n_tiles - 1;

  // ---- HBM -> LDS tile loads. Load r of wave w writes the 1 KiB block i = NW*r + w of the
  // tile (lane l -> chunk p = 64i + l: row p / DCH, physical chunk p % DCH) and fetches the
  // logical chunk the row's XOR swizzle maps there.
  uint32_t koff[S::LOADS];
#pragma unroll
  for (int r = 0; r < S::LOADS; ++r) {
    const int p = (S::NW * r + wave) * 64 + lane;
    const int row = p / S::DCH;
    const int pc = p % S::DCH;
    koff[r] = (uint32_t)(row * D * 2 + (pc ^ swz<D>(row)) * 16);
  }
  auto load_k = [&](int j, int slot) {
#pragma unroll
    for (int r = 0; r < S::LOADS; ++r)
      buffer_load16_to_lds(rk,
                           smem + S::K_SLOT0 + slot * S::TILE_BYTES + (S::NW * r + wave) * 1024,
                           koff[r], (uint32_t)j * BC * D * 2);
  };
  auto load_v = [&](int j, int slot) {
#pragma unroll
    for (int r = 0; r < S::LOADS; ++r)
      buffer_load16_to_lds(rv,
                           smem + S::V_SLOT0 + slot * S::TILE_BYTES + (S::NW * r + wave) * 1024,
                           koff[r], (uint32_t)j * BC * D * 2);
  };

  // ---- per-lane LDS read offsets (bytes within a tile). The swizzle depends on row bits 0-3
  // and permutes chunk bits 0-3 only, so 32-row block kb, 16-row step u and chunk bit 4
  // (+256 bytes, d = 256) become immediates.
  // K (A operand of S^T): row 32kb + kmap(l32), logical chunk 2kk + g.
  constexpr int KB8 = S::KK < 8 ? S::KK : 8;
  const int krow = kmap(l32);
  int kbase[KB8];
#pragma unroll
  for (int kk = 0; kk < KB8; ++kk) kbase[kk] = krow * D * 2 + ((2 * kk + g) ^ swz<D>(krow)) * 16;
  auto k_off = [&](int kb, int kk) { return kbase[kk % 8] + (kk / 8) * 256 + kb * 32 * D * 2; };
  // V^T fragments (A operand of O^T) via the transposing read: 16-lane group G = lane/16 covers
  // d rows c0 = 32cb + 16(G%2) .. +15 and k-slots 8g .. 8g+7 = keys 16u + 8g + 4h + (0..3).
  // Lane j of the group addresses key row 16u + 8g + 4h + j/4, columns c0 + 4(j%4) .. +3.
  constexpr int CB4 = S::CB < 4 ? S::CB : 4;
  const int jl = lane & 15;
  const int grp = lane >> 4;
  int vbase[CB4][2];
#pragma unroll
  for (int cb = 0; cb < CB4; ++cb)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = 8 * g + 4 * h + jl / 4;
      const int col = 32 * cb + 16 * (grp & 1) + 4 * (jl & 3);
      vbase[cb][h] =
          S::V_SLOT0 + row * D * 2 + (((col >> 3) ^ swz<D>(row)) * 16) + (col & 7) * 2;
    }
  auto v_off = [&](int cb, int u, int h) {
    return vbase[cb % 4][h] + (cb / 4) * 256 + 16 * u * D * 2;
  };

  // ---- Q^T fragments (B operand of S^T): lane holds q[my_q][16kk + 8g .. +7]; zeros past N;
  // the scale's sign applied (negated for a negative scale, zeroed for scale 0)
  u32x4_t qf[S::KK];
#pragma unroll
  for (int kk = 0; kk < S::KK; ++kk)
    qf[kk] = apply_sign(buffer_load16(rq, (uint32_t)my_q * D * 2 + (2 * kk + g) * 16, 0), qsign);

  // ---- accumulators and row statistics (per lane: query my_q, key half g)
  f32x16_t oacc[S::CB];
#pragma unroll
  for (int cb = 0; cb < S::CB; ++cb) oacc[cb] = f32x16_t{};
  float m_run;        // running max of scale*log2(e)*s (the row max may exceed it by <= 8)
  float l_f32 = 0.f;  // partial sum of p over this lane's keys
  float l_corr = 0.f; // masked tiles: sum of bf16(p) - p

  // hidden-key bias for tile j: -inf where key >= N or (causal) key > query
  auto tile_needs_mask = [&](int j) {
    const int key0 = j * BC;
    return (key0 + BC > N) || (CAUSAL && key0 + BC - 1 > q_wave0);
  };
  // (hidden iff key > key_lim: one compare per score)
  const int key_lim = CAUSAL ? min(my_q, N - 1) : N - 1;
  auto mask_bias = [&](int j, f32x16_t* s) {
#pragma unroll
    for (int kb = 0; kb < S::KB; ++kb) mask_keys(s[kb], j * BC + kb * 32 + 8 * g - key_lim);
  };
  // S^T tile j from K slot `slot`: KB 32-key blocks x 32 queries
  auto scores = [&](int slot, bool masked, int j, f32x16_t* s) {
    const unsigned char* kt = smem + S::K_SLOT0 + slot * S::TILE_BYTES;
    if (masked) mask_bias(j, s);
#pragma unroll
    for (int kk = 0; kk < S::KK; ++kk)
#pragma unroll
      for (int kb = 0; kb < S::KB; ++kb) {
        const u32x4_t a = *reinterpret_cast<const u32x4_t*>(kt + k_off(kb, kk));
        s[kb] = (kk == 0 && !masked) ? mfma32(a, qf[kk], f32x16_t{}) : mfma32(a, qf[kk], s[kb]);
      }
  };
  // 2*KB independent chains of 3-input maxima over the 16*KB scores of the lane
  auto row_max = [&](const f32x16_t* s) {
    constexpr int NC = 2 * S::KB;
    float a[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) a[c] = fmaxf(s[c / 2][8 * (c % 2)], s[c / 2][8 * (c % 2) + 1]);
#pragma unroll
    for (int i = 2; i < 8; i += 2)
#pragma unroll
      for (int c = 0; c < NC; ++c)
        a[c] = fmaxf(a[c], fmaxf(s[c / 2][8 * (c % 2) + i], s[c / 2][8 * (c % 2) + i + 1]));
    float m = fmaxf(a[0], a[1]);
#pragma unroll
    for (int c = 2; c < NC; c += 2) m = fmaxf(m, fmaxf(a[c], a[c + 1]));
    return max_xor32(m) * scale_log2;
  };
  // p = exp2(s*c - m) -> packed bf16 (the PV B operand); partial sum of p
  // dropout: keys 2m, 2m+1 are decided by the two halves of one word (the sums of p for the
  // normaliser and the LSE stay those of the undropped p)
  auto probs = [&](const f32x16_t* s, uint32_t (*pk)[8], int j) {
    const float neg_m = -m_run;
    // -0 is the identity of the fp32 add (-0 + x = x for every x), so the first add into each
    // partial sum folds away; +0 is not (+0 + -0 = +0), and the compiler keeps those adds
    float acc[4] = {-0.f, -0.f, -0.f, -0.f};
#pragma unroll
    for (int kb = 0; kb < S::KB; ++kb)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float p0 = fast_exp2(__builtin_fmaf(s[kb][2 * i], scale_log2, neg_m));
        const float p1 = fast_exp2(__builtin_fmaf(s[kb][2 * i + 1], scale_log2, neg_m));
        acc[(i & 1) * 2 + kb] += p0 + p1;
        if constexpr (DROP) {
          // registers 2i, 2i+1 of block kb hold keys j*BC + 32kb + 16(2i/8) + 8g + (2i%8) + 0, 1
          const int key = j * BC + 32 * kb + 16 * ((2 * i) / 8) + 8 * g + (2 * i) % 8;
          const uint32_t w = drop_word(drop_row, (uint32_t)key >> 1);
          pk[kb][i] = pack_bf16((w << 16) >= drop.thr ? p0 : 0.f, w >= drop.thr ? p1 : 0.f);
        } else {
          pk[kb][i] = pack_bf16(p0, p1);
        }
      }
    if constexpr (!DROP && D == 256) {
      // d = 256: each exponential between two plain VALU ops (FMAs of later scores, sums of
      // earlier p) instead of runs of eight (forward +3.0-3.1% at B2 H16 N4096; at d = 64 and
      // 128 the same order measured -1.4% to +0.3%)
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
#pragma unroll
      for (int i = 0; i < 16 * S::KB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x400, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
      }
    }
    return (acc[0] + acc[1]) + (acc[2] + acc[3]);
  };
  // masked tiles: l_corr += sum of bf16(p) - sum of p (after the PV MFMAs, off their path)
  auto bf16_correction = [&](uint32_t (*pk)[8], float tile_sum) {
    float b[2] = {-0.f, -0.f};  // (-0: see probs)
#pragma unroll
    for (int kb = 0; kb < S::KB; ++kb)
#pragma unroll
      for (int i = 0; i < 8; ++i) b[kb] = add_bf16_pair(b[kb], pk[kb][i]);
    l_corr += (b[0] + b[1]) - tile_sum;
  };
  // O^T += V^T P^T from V slot `slot`; MFMA u covers keys 16u .. 16u+15 = score block u/2,
  // registers 8(u%2) .. 8(u%2)+7
  auto pv = [&](int slot, uint32_t (*pk)[8]) {
    const unsigned char* vt = smem + slot * S::TILE_BYTES;  // (V_SLOT0 is in vbase)
#pragma unroll
    for (int u = 0; u < 2 * S::KB; ++u) {
      const u32x4_t b = {pk[u / 2][4 * (u % 2) + 0], pk[u / 2][4 * (u % 2) + 1],
                         pk[u / 2][4 * (u % 2) + 2], pk[u / 2][4 * (u % 2) + 3]};
#pragma unroll
      for (int cb = 0; cb < S::CB; ++cb) {
        const u32x2_t lo = lds_read_tr16(vt + v_off(cb, u, 0));
        const u32x2_t hi = lds_read_tr16(vt + v_off(cb, u, 1));
        const u32x4_t a = {lo[0], lo[1], hi[0], hi[1]};
        oacc[cb] = mfma32(a, b, oacc[cb]);
      }
    }
  };
  // raise the running max to the tile's max (rows whose max is already above keep alpha = 1)
  auto rescale_to = [&](float m_tile) {
    const float m_new = fmaxf(m_run, m_tile);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    l_f32 *= alpha;
    l_corr *= alpha;
#pragma unroll
    for (int cb = 0; cb < S::CB; ++cb) oacc[cb] *= alpha;
  };

  // ---- main loop over groups of TPB tiles: group g sits in ring half g % 2 (slots
  // TPB*(g%2) + i) and the next group streams into the other half while it is computed; one
  // barrier per group
  constexpr int TPB = S::TPB;
#pragma unroll
  for (int i = 0; i < TPB; ++i)
    if (i < n_tiles) {
      load_k(i, i);
      load_v(i, i);
    }
  wait_vmem();
  __syncthreads();
  m_run = -INFINITY;
  bool first = true;
  // tile j from slot `slot` (nothing for a wave whose rows all precede the tile's keys)
  auto tile = [&](auto slot_c, int j) {
    constexpr int slot = decltype(slot_c)::value;
    if (j <= wave_last) {
      f32x16_t s[S::KB];
      const bool masked = tile_needs_mask(j);
      if (masked) scores(slot, true, j, s);
      else scores(slot, false, j, s);
      uint32_t pk[S::KB][8];
      float tile_sum;
      if constexpr (S::KB == 2) {
        // deferred rescale without a max per tile: p is formed against the running max, and
        // only when some lane's partial sum exceeds 2^8 (so that a single p might) does the
        // wave take the tile's max, rescale and form p again (d <= 128: the scores stay live
        // until the check, which the d = 256 register budget has no room for)
        if (first) {
          m_run = row_max(s);  // tile 0 holds key 0, visible to every row: finite
          first = false;
        }
        tile_sum = probs(s, pk, j);
        if (__builtin_amdgcn_ballot_w64(!(tile_sum <= kRescaleSum)) != 0) {
          rescale_to(row_max(s));
          tile_sum = probs(s, pk, j);
        }
      } else {
        // d = 256: the tile's max first; rescale when it exceeds the running max by > 8
        const float m_tile = row_max(s);
        if (first) {
          m_run = m_tile;
          first = false;
        } else if (__builtin_amdgcn_ballot_w64(m_tile > m_run + kRescaleLog2) != 0) {
          rescale_to(m_tile);
        }
        tile_sum = probs(s, pk, j);
      }
      l_f32 += tile_sum;
      // raised priority while this wave issues its PV MFMAs: the other wave on the SIMD then
      // tends to run its softmax VALU work in between (measured +2-6%)
      __builtin_amdgcn_s_setprio(1);
      pv(slot, pk);
      __builtin_amdgcn_s_setprio(0);
      if (!DROP && masked) bf16_correction(pk, tile_sum);
    }
  };
  auto tile_group = [&](auto half_c, int j0) {
    constexpr int half = decltype(half_c)::value;
    // the other half held the previous group, whose readers all passed the barrier that ended it
    FA2_STAGE_SYNC();
#pragma unroll
    for (int i = 0; i < TPB; ++i)
      if (j0 + TPB + i < n_tiles) {
        load_k(j0 + TPB + i, (half ^ 1) * TPB + i);
        load_v(j0 + TPB + i, (half ^ 1) * TPB + i);
      }
    FA2_STAGE_SYNC();
    tile(std::integral_constant<int, half * TPB>{}, j0);
    if constexpr (TPB > 1) {
      if (j0 + 1 < n_tiles) tile(std::integral_constant<int, half * TPB + 1>{}, j0 + 1);
    }
    FA2_STAGE_SYNC();
    wait_vmem();
    __syncthreads();
  };
  for (int j0 = 0; j0 < n_tiles; j0 += 2 * TPB) {
    tile_group(std::integral_constant<int, 0>{}, j0);
    if (j0 + TPB < n_tiles) tile_group(std::integral_constant<int, 1>{}, j0 + TPB);
  }

  // ---- epilogue: deferred normalisation, bf16 output, LSE
  const float l_tot = sum_xor32(l_f32);
  const float l_o = sum_xor32(l_f32 + l_corr);
  const float inv = DROP ? fast_rcp(l_o) * drop.scale : fast_rcp(l_o);
  // (the loop ended with a barrier: the K/V tiles are free for the transpose)
  static_assert(S::NW * store_scratch_bytes(S::CB) <= S::SMEM, "transpose scratch");
  store_rows_via_lds<S::CB, D>(smem + wave * store_scratch_bytes(S::CB), oacc, inv, o + head_off,
                               my_q - l32, N, lane);
  if (my_q < N && g == 0) lse[(size_t)tc.bh * N + my_q] = (m_run + fast_log2(l_tot)) * kLn2;
}

template <int D, bool CAUSAL, bool DROP>
hipError_t launch_fwd_t(const FwdArgs& a) {
  const int n_qblocks = (a.N + FwdShape<D>::BR - 1) / FwdShape<D>::BR;
  const long long grid = (long long)n_qblocks * a.B * a.H;
  if (grid <= 0 || grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const DropParams drop{a.drop_k0, a.drop_k1, a.drop_thr, a.drop_scale};
  hipLaunchKernelGGL((fa2_fwd_kernel<D, CAUSAL, DROP>), dim3((unsigned)grid),
                     dim3(FwdShape<D>::THREADS),
                     0, a.stream, static_cast<const uint16_t*>(a.q),
                     static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.v),
                     static_cast<uint16_t*>(a.o), a.lse, a.N, n_qblocks, a.B * a.H,
                     causal_window(a.B * a.H, 4ll * a.N * D, n_qblocks, D == 64 ? 3 : 1,
                                   window_budget(D)), a.H,
                     a.H / a.Hkv, a.kv_bstride, a.scale_log2, OperandSign{a.q_and, a.q_xor},
                     drop);
  return hipGetLastError();
}

template <int D>
hipError_t launch_fwd_d(const FwdArgs& a) {
  if (a.dropout)
    return a.causal ? launch_fwd_t<D, true, true>(a) : launch_fwd_t<D, false, true>(a);
  return a.causal ? launch_fwd_t<D, true, false>(a) : launch_fwd_t<D, false, false>(a);
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a) {
  if (a.d == 64) return launch_fwd_d<64>(a);
  if (a.d == 256) return launch_fwd_d<256>(a);
  return launch_fwd_d<128>(a);
}

}  // namespace fa2
