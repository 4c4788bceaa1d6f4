// FlashAttention-2 backward for gfx950: dQ, dK, dV of O = softmax(scale Q K^T [+ causal]) V.
//
// The pages describe the backward as block-wise recomputation: recompute S and P for each
// block pair from Q, K and the saved softmax statistic, never store the N x N P or dP, and
// accumulate the gradients block by block (page "Flash Attention v2", sections "2. Backward
// Pass Computation" and "5. Gradient Accumulation"; a separate backward kernel, page
// "FlashAttention-2: Faster Attention with Better Parallelism and Work Partitioning"). The
// per-block arithmetic is the exact softmax gradient (the listing on the first page keeps only
// the diagonal of the softmax Jacobian; the full form is used):
//
//   P = exp(scale S - LSE),  D_i = sum_c dO_ic O_ic,  dS = P * (dO V^T - D),
//   dV = P^T dO,  dK = scale dS^T Q,  dQ = scale dS K.
//
// Deterministic (no atomics); the backward runs two kernels, dQ first:
//   fa2_bwd_dq_kernel    grid over (query block, head, batch), 256 queries at d = 128 (128 at
//                        d = 64 and 256): the forward's layout (lane = query). It first forms
//                        D_i = rowsum(dO_i * O_i) from the dO and O rows it loads and stores -D
//                        and LSE*log2(e) of its queries in the workspace; then it recomputes
//                        S^T and dP^T per key tile and accumulates dQ^T = K^T dS^T.
//   fa2_bwd_dkdv16_kernel grid over (key block, head, batch), 128 keys (64 at d = 256, and with
//                        dropout at d = 128): 32-query tiles of Q, dO, LSE*log2(e) and -D
//                        stream through LDS; each wave forms S and dP of its 16 or 32 keys
//                        with 16x16x32 MFMAs (lane = key) and accumulates its keys' dK, dV in
//                        registers.
//   fa2_bwd_pre_kernel   D and LSE*log2(e) alone (HBM-bound), for callers that want dK/dV
//                        without dQ.
// dK/dV and dQ each recompute S and dP; dQ's two recompute GEMMs are the price of avoiding
// atomic dQ accumulation. Without dropout the dP accumulators start at -D, so dP - D comes
// out of the MFMAs and dS is one multiply. Output tiles leave through LDS as whole row
// segments. With dropout (DROP) every kernel regenerates the keep bits it needs from the
// counter-based hash (fa2_device.hpp); dS = P * (Z * dP / P(keep) - D) and dV takes
// P * Z / P(keep).
#include <mutex>
#include <type_traits>

#include "fa2_device.hpp"
#include "fa2_launch.hpp"

namespace fa2 {

namespace {

constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;

// HBM -> LDS copy of a ROWS-row bf16 tile [ROWS][D] starting at byte `soff` of buffer `r`,
// into `dst` (row-major, swz<D>-swizzled 16-byte chunks, conflict-free for both the row-wise
// MFMA operand reads and the transposing reads), by a workgroup of NT threads. Load i of wave w
// writes the 1 KiB block (NT/64)i + w, lane l its 16 bytes at 16l: the physical chunk
// p = 64*block + l of the tile, which holds the logical chunk (p % DCH) ^ swz(row).
template <int D, int NT = kThreads, int ROWS = 64, bool SWZ16 = false>
struct TileLoader {
  static constexpr int DCH = D / 8;
  static constexpr int WAVES = NT / 64;
  static constexpr int LOADS = ROWS * D * 2 / (NT * 16);
  static_assert(LOADS >= 1 && LOADS * NT * 16 == ROWS * D * 2, "tile loader shape");
  uint32_t off[LOADS];
  int wave;
  __device__ __forceinline__ TileLoader(int wave_, int lane) : wave(wave_) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int p = (WAVES * i + wave) * 64 + lane;
      const int row = p / DCH;
      const int sw = SWZ16 ? swz16<D>(row) : swz<D>(row);
      off[i] = (uint32_t)(row * D * 2 + ((p % DCH) ^ sw) * 16);
    }
  }
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, unsigned char* dst,
                                       uint32_t soff) const {
#pragma unroll
    for (int i = 0; i < LOADS; ++i)
      buffer_load16_to_lds(r, dst + (WAVES * i + wave) * 1024, off[i], soff);
  }
};

// Per-lane byte offsets into a swizzled tile for the two read patterns. The swizzle permutes
// chunk bits 0-3 only, so at D = 256 chunk bit 4 (+256 bytes) is an immediate and 8 row and
// 4 x 2 transposing bases cover every read.
template <int D>
struct TileReads {
  static constexpr int KK = D / 16, CB = D / 32;
  static constexpr int KR = KK < 8 ? KK : 8, CR = CB < 4 ? CB : 4;
  int rbase[KR];     // row-wise operand reads: row 32*blk + kmap(l32), logical chunk 2kk + g
  int tbase[CR][2];  // transposing reads: row 16u + 8g + 4h + j/4, column 32cb + 16(G%2) + 4(j%4)
  __device__ __forceinline__ TileReads(int lane) {
    const int l32 = lane & 31, g = lane >> 5, jl = lane & 15, grp = lane >> 4;
    const int krow = kmap(l32);
#pragma unroll
    for (int kk = 0; kk < KR; ++kk) rbase[kk] = krow * D * 2 + ((2 * kk + g) ^ swz<D>(krow)) * 16;
#pragma unroll
    for (int cb = 0; cb < CR; ++cb)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int row = 8 * g + 4 * h + jl / 4;
        const int col = 32 * cb + 16 * (grp & 1) + 4 * (jl & 3);
        tbase[cb][h] = row * D * 2 + (((col >> 3) ^ swz<D>(row)) * 16) + (col & 7) * 2;
      }
  }
  __device__ __forceinline__ int row_off(int blk, int kk) const {
    return rbase[kk % 8] + (kk / 8) * 256 + blk * 32 * D * 2;
  }
  __device__ __forceinline__ int tr_off(int cb, int u, int h) const {
    return tbase[cb % 4][h] + (cb / 4) * 256 + 16 * u * D * 2;
  }
};

// 8 bf16 of a 32x32x16 MFMA operand as two transposing reads (k-slots 0..3 and 4..7).
__device__ __forceinline__ u32x4_t tr_operand(const unsigned char* tile, int off_h0, int off_h1) {
  const u32x2_t lo = lds_read_tr16(tile + off_h0);
  const u32x2_t hi = lds_read_tr16(tile + off_h1);
  return u32x4_t{lo[0], lo[1], hi[0], hi[1]};
}

// ---------------------------------------------------------------------------------------
// D = rowsum(dO * O): D/8 lanes per row, 16 bytes each, reduced across the row's lanes. It is
// stored negated (-D: the dK/dV kernel starts its dP accumulators there, so dP - D comes out of
// the MFMAs). The same pass stores LSE * log2(e), the form the other two kernels subtract
// inside exp2.
template <int D>
__global__ __launch_bounds__(kThreads) void fa2_bwd_pre_kernel(const uint16_t* __restrict__ o,
                                                               const uint16_t* __restrict__ dout,
                                                               const float* __restrict__ lse,
                                                               float* __restrict__ delta,
                                                               float* __restrict__ lse2,
                                                               long long rows) {
  constexpr int TPR = D / 8;
  const long long t = (long long)blockIdx.x * kThreads + threadIdx.x;
  const long long row = t / TPR;
  const int c = (int)(t % TPR);
  float acc = 0.f;
  if (row < rows) {
    const u32x4_t a = *reinterpret_cast<const u32x4_t*>(o + row * D + c * 8);
    const u32x4_t b = *reinterpret_cast<const u32x4_t*>(dout + row * D + c * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      acc += bf16_lo(a[e]) * bf16_lo(b[e]) + bf16_hi(a[e]) * bf16_hi(b[e]);
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && c == 0) {
    delta[row] = -acc;
    lse2[row] = lse[row] * kLog2e;
  }
}

// ---------------------------------------------------------------------------------------
// Position in a dK/dV workgroup's walk over (query head, query tile) steps: head qh0 + gi,
// tile it, advanced one step at a time (no integer division per step).
struct StepPos {
  int gi, it;
  int it0, it_end;
  __device__ __forceinline__ StepPos(int t, int nt, int qt_begin)
      : gi(t / nt), it(qt_begin + t % nt), it0(qt_begin), it_end(qt_begin + nt) {}
  __device__ __forceinline__ void next() {
    if (++it == it_end) {
      it = it0;
      ++gi;
    }
  }
};

// ---------------------------------------------------------------------------------------
// Dropout in the dK/dV kernels (lane = key, registers = queries). The row keys of a query tile
// go to LDS with the tile (one hash per query, by one wave); the two lanes of a key pair (lanes
// 2m', 2m'+1 hold keys 2m, 2m+1) need the same word per query, so each hashes half of its 16
// queries and takes the other half from its neighbour by DPP, then picks its 16-bit half.

// Row key of query row0 + lane of query head qh, stored at rk[lane].
__device__ __forceinline__ void store_row_key(unsigned char* rk, const DropParams& drop, int qh,
                                              int row0, int lane) {
  const uint32_t a = drop_head_key(drop, (uint32_t)qh);
  reinterpret_cast<uint32_t*>(rk)[lane] = pcg_hash(a ^ (uint32_t)(row0 + lane));
}

// ---------------------------------------------------------------------------------------
// dK, dV with 16-key MFMA blocks (v_mfma_f32_16x16x32_bf16). Workgroup = 4 waves over 64*KP
// keys, one wave per SIMD, and several workgroups per CU (3 at d = 64, 2 at d = 128 and 256;
// with dropout 2 at d = 128 and 1 at d = 256, where the keep words and -D take the registers of a
// second wave), so each SIMD runs waves of independent workgroups. With KP = 1 (d = 256, and
// with dropout at d = 128) a wave keeps its 16
// keys' K and V fragments in registers (loaded once, the scale's sign applied to K) and its
// dK^T, dV^T accumulators (d x 16 keys); 32-query tiles of Q and dO with their LSE*log2(e) and -D stream
// through a 2-stage LDS ring (swz16 layout). Per tile, S = Q K^T and dP = dO V^T come out as two
// 16-query blocks with lane = key (query order: block b, register r of lane group g is query
// 16b + 4g + r), so the packed P and dS are directly the B operands of dV^T += dO^T P and
// dK^T += Q^T dS over the tile's 32 queries, whose A operands (dO^T, Q^T) come from transposing
// reads of the same tiles. S is formed once per (key, query) pair and dK, dV share it (a split
// into dK waves and dV waves would form it twice); the K/V operands come from registers.
// KP = 2 (d = 64, 128): each wave takes two 16-key sub-blocks (32 keys) that share every Q and
// dO operand read, which halves the LDS reads per MFMA of those operands; the 128 keys' K rows
// then stay in LDS (read per step) and only V's fragments live in registers, and 3 (d = 64) or
// 2 (d = 128) workgroups of 4 waves share a CU, each SIMD interleaving independent workgroups.
template <int D, int KP = 1, bool DROP = false>
struct Kv16Shape {
  static constexpr int NW = 4, THREADS = 256, BQ = 32;
  static constexpr int BK = 64 * KP;                            // keys per workgroup
  static constexpr int OCC =
      KP > 1 ? (D == 64 ? 3 : 2) : (D == 64 ? 4 : (D == 128 ? (DROP ? 2 : 3) : (DROP ? 1 : 2)));
  static constexpr int KS = D / 32;                             // k-steps of S and dP
  static constexpr int DB = D / 16;                             // 16-row blocks of dV^T, dK^T
  static constexpr int TILE = BQ * D * 2;
  // LSE*log2(e) of the 32 queries, then -D, then (dropout) their row keys; 512 bytes with
  // dropout, so that every tile starts on a 256-byte bank window
  static constexpr int STATS = DROP ? 512 : 2 * BQ * 4;
  static constexpr int STAGE = 2 * TILE + STATS;
  static constexpr int KRES0 = 2 * STAGE;                // resident K rows (KP > 1)
  static constexpr int KRES = KP > 1 ? BK * D * 2 : 0;
  static constexpr int SMEM = KRES0 + KRES;
};

// The 16*KP x D tile of a wave's dK^T or dV^T accumulators (lane = key 16kp + l%16, columns
// 16blk + 4(l/16) + (0..3)) times `mul`, as bf16 into rows row0 .. row0+16KP-1 of `out` (row
// stride D; rows >= n_rows skipped) through `scratch` (LDS that only this wave uses,
// rows16_scratch_bytes bytes, rows padded by 16 bytes: the 8-byte writes of 16 rows x 2 column
// groups fall in distinct banks), so each global store writes whole row segments, 16 bytes per
// lane, rather than 8 bytes in each of 16 rows. A wave's LDS accesses complete in order, so the
// reads see the writes and the next call's writes follow this call's reads.
template <int D, int KP>
constexpr int rows16_scratch_bytes() { return 16 * KP * (D * 2 + 16); }
template <int D, int KP>
__device__ __forceinline__ void store_rows16_via_lds(unsigned char* scratch,
                                                     const f32x4_t (*acc)[D / 16], float mul,
                                                     uint16_t* out, int row0, int n_rows,
                                                     int lane) {
  constexpr int PITCH = D * 2 + 16;
  constexpr int CH = D / 8, RPI = 64 / CH;  // 16-byte chunks per row, rows per store
  const int kl = lane & 15, g = lane >> 4;
#pragma unroll
  for (int kp = 0; kp < KP; ++kp)
#pragma unroll
    for (int blk = 0; blk < D / 16; ++blk)
      *reinterpret_cast<u32x2_t*>(scratch + (16 * kp + kl) * PITCH + (16 * blk + 4 * g) * 2) =
          u32x2_t{pack_bf16(acc[kp][blk][0] * mul, acc[kp][blk][1] * mul),
                  pack_bf16(acc[kp][blk][2] * mul, acc[kp][blk][3] * mul)};
#pragma unroll
  for (int i = 0; i < 16 * KP / RPI; ++i) {
    const int rr = i * RPI + lane / CH, ch = lane % CH;
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(scratch + rr * PITCH + ch * 16);
    if (row0 + rr < n_rows) *reinterpret_cast<u32x4_t*>(out + (size_t)(row0 + rr) * D + ch * 8) = v;
  }
}
// The dK/dV kernel writes its rows through LDS: fwd+bwd step at B4 H16 N2048 d128 +1.9% causal,
// +1.3% non-causal; at d = 64 (B8 H32 N2048) +0.8-1.4% and d = 256 (B2 H16 N4096) +0.4-0.8%, once
// the epilogue's addresses were kept from being computed before the key loop (held across it, they
// had made the compiler spill 4 and 12 registers in the causal kernels: -2.7% and -7.9%).
#ifndef FA2_DKDV16_LDS_EPILOGUE
#define FA2_DKDV16_LDS_EPILOGUE 1
#endif
#ifndef FA2_DKDV16_LDS_EPILOGUE_MAX_D
#define FA2_DKDV16_LDS_EPILOGUE_MAX_D 256
#endif

template <int D, bool CAUSAL, int KP, bool DROP>
__global__ __launch_bounds__(256, (Kv16Shape<D, KP, DROP>::OCC))
__attribute__((amdgpu_waves_per_eu(Kv16Shape<D, KP, DROP>::OCC, Kv16Shape<D, KP, DROP>::OCC))) void
fa2_bwd_dkdv16_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                      const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
                      const float* __restrict__ lse2, const float* __restrict__ delta,
                      uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int N, int n_kblocks,
                      int bh_count, int window, int n_qheads, int group, long long kv_bstride,
                      float scale_log2, float scale, OperandSign ksign, DropParams drop,
                      float* __restrict__ part, int split) {
  using S = Kv16Shape<D, KP, DROP>;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[S::SMEM];
  static_assert(4 * rows16_scratch_bytes<D, KP>() <= S::SMEM, "output scratch");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kl = lane & 15;  // this lane's key within each 16-key sub-block
  const int g = lane >> 4;   // lane group: queries 4g .. 4g+3 of each 16-query block

  // causal: key block 0 sees every query tile, so ascending order is longest first
  const TileCoord tc = schedule_tile<CAUSAL ? Order::kLongAscending : Order::kHeadMajor>(
      blockIdx.x, n_kblocks, bh_count, window);
  // tc.bh = (batch * Hkv + K/V head) * split + part
  const int sj = tc.bh % split;
  const int bhkv = tc.bh / split;
  const int n_kvheads = n_qheads / group;
  const int b_idx = bhkv / n_kvheads;
  const int kvh = bhkv - b_idx * n_kvheads;
  const int qh0 = b_idx * n_qheads + kvh * group;
  const size_t head_off =  // K, V, dK, dV
      (size_t)b_idx * (size_t)kv_bstride + (size_t)kvh * (size_t)N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const int key_b0 = tc.qb * S::BK;
  const int key_w0 = key_b0 + wave * 16 * KP;  // sub-block kp: keys key_w0 + 16kp + (0..15)

  // per-lane LDS offsets within a tile (and the resident K rows): operand rows (row 16b + kl,
  // logical chunk 4ks + g) at row_base + 16*D*2*b + ((64*ks) ^ row_x); transposing reads
  // (queries 4g + 16h + j/4, d columns 16blk + 4(j%4)) at tr_base[h] + ((32*blk) ^ tr_x[h])
  const int row_base = kl * D * 2;
  const int row_x = 16 * (g ^ swz16<D>(kl));
  int tr_base[2], tr_x[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int j = lane & 15;
    const int row = 4 * g + 16 * h + (j >> 2);
    tr_base[h] = row * D * 2 + 8 * (j & 1);
    tr_x[h] = 16 * (((j & 3) >> 1) ^ swz16<D>(row));
  }

  // V fragments (B operands of dP = dO V^T) of the wave's keys, and K's (of S = Q K^T) when they
  // live in registers: lane holds row key_w0 + 16kp + kl, columns 32ks + 8g .. +7 (zeros past N)
  u32x4_t kf[KP == 1 ? S::KS : 1], vf[KP][S::KS];
  {
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(v + head_off, head_bytes);
#pragma unroll
    for (int kp = 0; kp < KP; ++kp)
#pragma unroll
      for (int ks = 0; ks < S::KS; ++ks)
        vf[kp][ks] = buffer_load16(
            rv, (uint32_t)(key_w0 + 16 * kp + kl) * D * 2 + (32 * ks + 8 * g) * 2, 0);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + head_off, head_bytes);
    if constexpr (KP == 1) {
#pragma unroll
      for (int ks = 0; ks < S::KS; ++ks)
        kf[ks] = apply_sign(
            buffer_load16(rk, (uint32_t)(key_w0 + kl) * D * 2 + (32 * ks + 8 * g) * 2, 0), ksign);
    } else {
      // the workgroup's K rows into LDS (swz16 layout, rows = keys)
      const TileLoader<D, S::THREADS, S::BK, true> kld(wave, lane);
      kld.load(rk, smem + S::KRES0, (uint32_t)key_b0 * D * 2);
    }
  }

  const int n_qt = (N + S::BQ - 1) / S::BQ;
  const int qt_begin = CAUSAL ? key_b0 / S::BQ : 0;
  const int nt = n_qt - qt_begin;
  const long long n_all = (long long)group * nt;
  const int t_begin = (int)(n_all * sj / split);
  const int n_steps = (int)(n_all * (sj + 1) / split) - t_begin;
  const TileLoader<D, S::THREADS, S::BQ, true> ld(wave, lane);

  StepPos ldpos(t_begin, nt, qt_begin);  // the next tile to load (loads go in step order)
  int ld_head = -1;
  __amdgpu_buffer_rsrc_t rq, rdo, rl, rd;
  auto load_stage = [&](int stage) {
    const int gi = ldpos.gi;
    const int it = ldpos.it;
    ldpos.next();
    if (gi != ld_head) {
      ld_head = gi;
      const size_t qoff = (size_t)(qh0 + gi) * (size_t)N * D;
      rq = make_rsrc(q + qoff, head_bytes);
      rdo = make_rsrc(dout + qoff, head_bytes);
      rl = make_rsrc(lse2 + (size_t)(qh0 + gi) * N, (uint32_t)N * 4);
      rd = make_rsrc(delta + (size_t)(qh0 + gi) * N, (uint32_t)N * 4);
    }
    unsigned char* st = smem + stage * S::STAGE;
    const uint32_t soff = (uint32_t)it * S::BQ * D * 2;
    ld.load(rq, st, soff);
    ld.load(rdo, st + S::TILE, soff);
    // LSE*log2(e) and -D of the tile's 32 queries (128 bytes each): 8 lanes of waves 0 and 1
    unsigned char* sst = st + 2 * S::TILE;
    if (wave == 0) {
      if (lane < 8) buffer_load16_to_lds(rl, sst, (uint32_t)lane * 16, (uint32_t)it * S::BQ * 4);
    } else if (wave == 1) {
      if (lane < 8)
        buffer_load16_to_lds(rd, sst + S::BQ * 4, (uint32_t)lane * 16, (uint32_t)it * S::BQ * 4);
    } else if (DROP && wave == 2) {
      if (lane < S::BQ) store_row_key(sst + 2 * S::BQ * 4, drop, qh0 + gi, it * S::BQ, lane);
    }
  };

  f32x4_t dkacc[KP][S::DB], dvacc[KP][S::DB];
#pragma unroll
  for (int kp = 0; kp < KP; ++kp)
#pragma unroll
    for (int b = 0; b < S::DB; ++b) {
      dkacc[kp][b] = f32x4_t{};
      dvacc[kp][b] = f32x4_t{};
    }

  if (n_steps > 0) load_stage(0);
  wait_vmem();
  __syncthreads();
  if constexpr (KP > 1) {
    if (ksign.and_mask != ~0u || ksign.xor_mask != 0u) {
      // a scale <= 0: its sign goes into the resident K rows, once (see OperandSign)
      for (int i = tid * 16; i < S::KRES; i += S::THREADS * 16)
        *reinterpret_cast<u32x4_t*>(smem + S::KRES0 + i) =
            apply_sign(*reinterpret_cast<const u32x4_t*>(smem + S::KRES0 + i), ksign);
      __syncthreads();
    }
  }
  // this wave's first K row in LDS (sub-block kp adds 16 rows)
  const unsigned char* kres = smem + S::KRES0 + (size_t)wave * 16 * KP * D * 2;

  StepPos cur(t_begin, nt, qt_begin);  // the tile of the current step
  auto step = [&](auto stage_c, int t) {
    constexpr int stage = decltype(stage_c)::value;
    FA2_STAGE_SYNC();
    if (t + 1 < n_steps) load_stage(stage ^ 1);
    FA2_STAGE_SYNC();
    const int it = cur.it;
    cur.next();
    const int q0 = it * S::BQ;
    // every query of the tile precedes every key of the wave: fully masked
    const bool skip = CAUSAL && (q0 + S::BQ - 1 < key_w0);
    if (!skip) {
      const unsigned char* tq = smem + stage * S::STAGE;
      const unsigned char* tdo = tq + S::TILE;
      const unsigned char* ts = tq + 2 * S::TILE;
      // LSE*log2(e) and -D of this lane's queries 16b + 4g + (0..3)
      const f32x4_t lsv[2] = {*reinterpret_cast<const f32x4_t*>(ts + 16 * g),
                              *reinterpret_cast<const f32x4_t*>(ts + 64 + 16 * g)};
      // (with dropout -D is read after the score MFMAs, where it is used)
      f32x4_t ndv[2] = {};
      if constexpr (!DROP) {
        ndv[0] = *reinterpret_cast<const f32x4_t*>(ts + S::BQ * 4 + 16 * g);
        ndv[1] = *reinterpret_cast<const f32x4_t*>(ts + S::BQ * 4 + 64 + 16 * g);
      }
      // dP starts at -D, so the MFMAs leave dP - D
      f32x4_t sacc[KP][2], dpacc[KP][2];
#pragma unroll
      for (int kp = 0; kp < KP; ++kp)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          sacc[kp][b] = f32x4_t{};
          dpacc[kp][b] = DROP ? f32x4_t{} : ndv[b];
        }
#pragma unroll
      for (int ks = 0; ks < S::KS; ++ks) {
        const int off = row_base + ((64 * ks) ^ row_x);
        u32x4_t kk[KP];
        if constexpr (KP == 1) {
          kk[0] = kf[ks];
        } else {
#pragma unroll
          for (int kp = 0; kp < KP; ++kp)
            kk[kp] = *reinterpret_cast<const u32x4_t*>(kres + off + kp * 16 * D * 2);
        }
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const u32x4_t aq = *reinterpret_cast<const u32x4_t*>(tq + off + b * 16 * D * 2);
          const u32x4_t ad = *reinterpret_cast<const u32x4_t*>(tdo + off + b * 16 * D * 2);
#pragma unroll
          for (int kp = 0; kp < KP; ++kp) {
            sacc[kp][b] = mfma16(aq, kk[kp], sacc[kp][b]);
            dpacc[kp][b] = mfma16(ad, vf[kp][ks], dpacc[kp][b]);
          }
        }
      }
      // hidden pairs (query past N, or causal query before the key) get S = -inf, so P = 0
      const bool masked = (q0 + S::BQ > N) || (CAUSAL && q0 < key_w0 + 16 * KP - 1);
      if (masked) {
#pragma unroll
        for (int kp = 0; kp < KP; ++kp)
#pragma unroll
          for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int qq = q0 + 16 * b + 4 * g + r;
              if (qq >= N || (CAUSAL && qq < key_w0 + 16 * kp + kl)) sacc[kp][b][r] = -INFINITY;
            }
      }
      // P = exp2(S*c - LSE*log2(e)), dS = P * (dP - D), packed as the B operands (queries
      // 8g .. 8g+7 of the MFMA's k range = block 0 registers, then block 1 registers)
      u32x4_t bp[KP], bs[KP];
      // dropout: the words of this lane's 8 queries (registers of blocks 0, 1) and its key pair.
      // The two lanes of a pair (kl even, odd: keys 2m, 2m+1) hold the same queries: the even
      // lane hashes block 0's four, the odd lane block 1's, each takes the other four from its
      // neighbour (DPP), and a byte permute moves the key's 16 bits to the top (low half for the
      // even key, high half for the odd one), zeros below.
      const int odd = kl & 1;
      u32x4_t rkeys = {};
      if constexpr (DROP) {
        rkeys = *reinterpret_cast<const u32x4_t*>(ts + 2 * S::BQ * 4 + 64 * odd + 16 * g);
        ndv[0] = *reinterpret_cast<const f32x4_t*>(ts + S::BQ * 4 + 16 * g);
        ndv[1] = *reinterpret_cast<const f32x4_t*>(ts + S::BQ * 4 + 64 + 16 * g);
      }
#pragma unroll
      for (int kp = 0; kp < KP; ++kp) {
        float pv[8], dsv[8];
        uint32_t dw[2][4];
        if constexpr (DROP) {
          const uint32_t pair = (uint32_t)((key_w0 + 16 * kp + kl) >> 1) * kDropKeyMul;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint32_t w = pcg_hash(rkeys[r] ^ pair);
            const uint32_t x = swap_adjacent_lanes(w);
            dw[0][r] = __builtin_amdgcn_perm(x, w, odd ? 0x07060C0Cu : 0x01000C0Cu);
            dw[1][r] = __builtin_amdgcn_perm(x, w, odd ? 0x03020C0Cu : 0x05040C0Cu);
          }
        }
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float p = fast_exp2(__builtin_fmaf(sacc[kp][b][r], scale_log2, -lsv[b][r]));
            if constexpr (DROP) {
              // kept with its 1/P(keep) scale, or 0: dV takes P*Z, dS = P*(Z*dP - D)
              const float zs = dw[b][r] >= drop.thr ? drop.scale : 0.f;
              pv[4 * b + r] = p * zs;
              dsv[4 * b + r] = p * __builtin_fmaf(dpacc[kp][b][r], zs, ndv[b][r]);
            } else {
              pv[4 * b + r] = p;
              dsv[4 * b + r] = p * dpacc[kp][b][r];
            }
          }
        bp[kp] = u32x4_t{pack_bf16(pv[0], pv[1]), pack_bf16(pv[2], pv[3]), pack_bf16(pv[4], pv[5]),
                         pack_bf16(pv[6], pv[7])};
        bs[kp] = u32x4_t{pack_bf16(dsv[0], dsv[1]), pack_bf16(dsv[2], dsv[3]),
                         pack_bf16(dsv[4], dsv[5]), pack_bf16(dsv[6], dsv[7])};
      }
      // raised priority while the wave issues its dV/dK MFMAs
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int blk = 0; blk < S::DB; ++blk) {
        const int o0 = tr_base[0] + ((32 * blk) ^ tr_x[0]);
        const int o1 = tr_base[1] + ((32 * blk) ^ tr_x[1]);
        const u32x4_t ao = tr_operand(tdo, o0, o1);
        const u32x4_t aq = tr_operand(tq, o0, o1);
#pragma unroll
        for (int kp = 0; kp < KP; ++kp) {
          dvacc[kp][blk] = mfma16(ao, bp[kp], dvacc[kp][blk]);
          dkacc[kp][blk] = mfma16(aq, bs[kp], dkacc[kp][blk]);
        }
      }
      __builtin_amdgcn_s_setprio(0);
    }
    FA2_STAGE_SYNC();
    wait_vmem();
    __syncthreads();
  };
  for (int t = 0; t < n_steps; t += 2) {
    step(std::integral_constant<int, 0>{}, t);
    if (t + 1 < n_steps) step(std::integral_constant<int, 1>{}, t + 1);
  }

  // dK = scale * dK_acc, dV = dV_acc: lane holds key key_w0 + 16kp + kl, d columns
  // 16blk + 4g + (0..3)
  if (FA2_DKDV16_LDS_EPILOGUE && D <= FA2_DKDV16_LDS_EPILOGUE_MAX_D && part == nullptr) {
    // whole rows through LDS (the loop ended with a barrier: ring and resident K rows are free).
    // The lane index passes through an empty asm statement so that the compiler cannot compute
    // the epilogue's addresses before the loop and hold them across it
    int lane_e = lane;
    asm volatile("" : "+v"(lane_e));
    unsigned char* sc = smem + wave * rows16_scratch_bytes<D, KP>();
    store_rows16_via_lds<D, KP>(sc, dkacc, scale, dk + head_off, key_w0, N, lane_e);
    store_rows16_via_lds<D, KP>(sc, dvacc, 1.f, dv + head_off, key_w0, N, lane_e);
    return;
  }
#pragma unroll
  for (int kp = 0; kp < KP; ++kp) {
    const int my_key = key_w0 + 16 * kp + kl;
    if (my_key >= N) continue;
    if (part == nullptr) {
      uint16_t* dkrow = dk + head_off + (size_t)my_key * D + 4 * g;
      uint16_t* dvrow = dv + head_off + (size_t)my_key * D + 4 * g;
#pragma unroll
      for (int blk = 0; blk < S::DB; ++blk) {
        *reinterpret_cast<u32x2_t*>(dkrow + 16 * blk) =
            u32x2_t{pack_bf16(dkacc[kp][blk][0] * scale, dkacc[kp][blk][1] * scale),
                    pack_bf16(dkacc[kp][blk][2] * scale, dkacc[kp][blk][3] * scale)};
        *reinterpret_cast<u32x2_t*>(dvrow + 16 * blk) =
            u32x2_t{pack_bf16(dvacc[kp][blk][0], dvacc[kp][blk][1]),
                    pack_bf16(dvacc[kp][blk][2], dvacc[kp][blk][3])};
      }
    } else {
      const size_t n_bhkv = (size_t)(bh_count / split);
      float* pk = part + (size_t)sj * n_bhkv * N * D + (size_t)bhkv * N * D +
                  (size_t)my_key * D + 4 * g;
      float* pvv = part + ((size_t)split + sj) * n_bhkv * N * D + (size_t)bhkv * N * D +
                   (size_t)my_key * D + 4 * g;
#pragma unroll
      for (int blk = 0; blk < S::DB; ++blk) {
        *reinterpret_cast<f32x4_t*>(pk + 16 * blk) = dkacc[kp][blk] * scale;
        *reinterpret_cast<f32x4_t*>(pvv + 16 * blk) = dvacc[kp][blk];
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// dQ. Workgroup = DqShape<D>::NW waves x 32 queries (lane = query, as in the forward); key
// tiles of 64 (32 at d = 256). S^T = K Q^T and dP^T = V dO^T from row-wise K/V tile reads
// with Q^T/dO^T fragments held in VGPRs; dQ^T += K^T dS^T with K^T fragments from
// transposing reads of the same K tile.
//  * d = 128: as in the forward, 8 waves (256 queries, one workgroup per CU) share each K/V
//    tile, halving the L2 -> LDS traffic per FLOP of 4 waves (dQ at B4 H16 N2048 d128 causal:
//    109 -> 105 us);
//  * d = 64: 4 waves, three workgroups per CU;
//  * d = 256: the resident Q^T and dO^T fragments and the dQ^T accumulators take 256 registers,
//    so 4 waves with one wave per SIMD (512 registers) accumulate whole rows in one launch. Two
//    launches of half the columns at two waves per SIMD each recomputed S and dP, 1.7x the
//    MFMAs, and took 1.47x as long (B2 H16 N4096 causal: 0.61 -> 0.41 ms).
template <int D>
struct DqShape {
  static constexpr int NW = D == 128 ? 8 : 4;  // waves per workgroup
  static constexpr int OCC = D == 256 ? 1 : 2; // waves per SIMD the kernel is compiled for
  static constexpr int BR = 32 * NW;           // query rows per workgroup
  static constexpr int THREADS = 64 * NW;
};

// Largest head dimension whose dQ kernel keeps separate code for masked and unmasked tiles
// (unmasked ones then start S at a constant zero instead of clearing 32 registers per tile):
// fwd+bwd step at B4 H16 N2048 d128 +0.5% causal, +1.2% without the mask; at d = 256 the
// second copy measured -0.5% on the B2 H16 N4096 steps.
#ifndef FA2_DQ_SPLIT_MAX_D
#define FA2_DQ_SPLIT_MAX_D 128
#endif
template <int D, bool CAUSAL, bool DROP>
__global__ __launch_bounds__((DqShape<D>::THREADS), (DqShape<D>::OCC)) void fa2_bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ o,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse, float* __restrict__ lse2,
    float* __restrict__ delta, uint16_t* __restrict__ dq, int N, int n_qblocks, int bh_count,
    int window, int n_qheads, int group, long long kv_bstride, float scale_log2, float scale,
    OperandSign qsign, DropParams drop) {
  constexpr int KK = D / 16, CB = D / 32;
  constexpr int BC = D == 256 ? 32 : 64;   // keys per tile
  constexpr int KB = BC / 32;              // 32-key MFMA blocks per tile
  constexpr int TILE = BC * D * 2;
  constexpr int STAGE = 2 * TILE;  // K, V
  constexpr int NW = DqShape<D>::NW;
  constexpr int SCRATCH = NW * store_scratch_bytes(CB);  // output tiles through LDS
  constexpr int SMEM = 2 * STAGE > SCRATCH ? 2 * STAGE : SCRATCH;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[SMEM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int g = lane >> 5;

  const TileCoord tc = schedule_tile<CAUSAL ? Order::kLongDescending : Order::kHeadMajor>(
      blockIdx.x, n_qblocks, bh_count, window);
  const size_t head_off = (size_t)tc.bh * (size_t)N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(q + head_off, head_bytes);
  // K/V head of this query head (grouped heads share one; batch stride may be packed)
  const int b_idx = tc.bh / n_qheads;
  const size_t kv_off = (size_t)b_idx * (size_t)kv_bstride +
                        (size_t)((tc.bh - b_idx * n_qheads) / group) * (size_t)N * D;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + kv_off, head_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(v + kv_off, head_bytes);
  const __amdgpu_buffer_rsrc_t rdo = make_rsrc(dout + head_off, head_bytes);

  const int q_block0 = tc.qb * DqShape<D>::BR;
  const int q_wave0 = q_block0 + wave * 32;
  const int my_q = q_wave0 + l32;
  const uint32_t drop_row =  // dropout: row key of this lane's query
      DROP ? pcg_hash(drop_head_key(drop, (uint32_t)tc.bh) ^ (uint32_t)my_q) : 0u;
  const bool valid_q = my_q < N;
  // masked tiles hide the keys above key_lim (the causal diagonal and the ragged tail)
  const int key_lim = CAUSAL ? min(my_q, N - 1) : N - 1;

  // Q and dO fragments (B operands of S^T and dP^T): lane holds row my_q, columns
  // 16kk + 8g .. +7; the O fragments of the same columns give this lane's half of
  // D = rowsum(dO * O), the other half is in lane l^32.
  u32x4_t qf[KK], dof[KK];
  float dpart = 0.f;
  {
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(o + head_off, head_bytes);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      // the scale's sign applied to Q (negated for a negative scale, zeroed for scale 0)
      qf[kk] = apply_sign(buffer_load16(rq, (uint32_t)my_q * D * 2 + (2 * kk + g) * 16, 0), qsign);
      dof[kk] = buffer_load16(rdo, (uint32_t)my_q * D * 2 + (2 * kk + g) * 16, 0);
    }
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const u32x4_t of = buffer_load16(ro, (uint32_t)my_q * D * 2 + (2 * kk + g) * 16, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        dpart += bf16_lo(dof[kk][e]) * bf16_lo(of[e]) + bf16_hi(dof[kk][e]) * bf16_hi(of[e]);
    }
  }
  const float dsum = sum_xor32(dpart);
  // padded queries get LSE = +inf, hence P = 0
  const float lse_q = valid_q ? lse[(size_t)tc.bh * N + my_q] * kLog2e : INFINITY;
  const float dlt = valid_q ? dsum : 0.f;
  // -D and LSE*log2(e) of this block's queries go to the workspace for the dK/dV kernel
  if (valid_q && g == 0) {
    delta[(size_t)tc.bh * N + my_q] = -dlt;
    lse2[(size_t)tc.bh * N + my_q] = lse_q;
  }

  int n_tiles = (N + BC - 1) / BC;
  if (CAUSAL) n_tiles = min(N - 1, q_block0 + DqShape<D>::BR - 1) / BC + 1;
  const int wave_last = CAUSAL ? min(n_tiles - 1, (q_wave0 + 31) / BC) : n_tiles - 1;

  const TileLoader<D, DqShape<D>::THREADS, BC> ld(wave, lane);
  const TileReads<D> rd_off(lane);
  auto load_stage = [&](int j, int stage) {
    unsigned char* st = smem + stage * STAGE;
    const uint32_t soff = (uint32_t)j * BC * D * 2;
    ld.load(rk, st, soff);
    ld.load(rv, st + TILE, soff);
  };

  f32x16_t dqacc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) dqacc[cb] = f32x16_t{};
  // without dropout (and for d <= 128, where the 16 registers fit) the dP^T chains start at -D
  // (all 16 registers of a lane are its query), so the MFMAs leave dP - D
  constexpr bool kInitD = !DROP && D <= 128;
  f32x16_t dp_init;
#pragma unroll
  for (int i = 0; i < 16; ++i) dp_init[i] = kInitD ? -dlt : 0.f;

  load_stage(0, 0);
  wait_vmem();
  __syncthreads();

  // unrolled by two below: the stage is a compile-time constant
  auto step = [&](auto stage_c, int j) {
    constexpr int stage = decltype(stage_c)::value;
    FA2_STAGE_SYNC();
    if (j + 1 < n_tiles) load_stage(j + 1, stage ^ 1);
    FA2_STAGE_SYNC();
    if (j <= wave_last) {
      const unsigned char* tk = smem + stage * STAGE;
      const unsigned char* tv = tk + TILE;
      const int key0 = j * BC;
      const bool masked = (key0 + BC > N) || (CAUSAL && key0 + BC - 1 > q_wave0);
      f32x16_t s[KB], dp[KB];
      // S^T and dP^T. MODE 0: unmasked tile, S starts at a constant zero (no register clears);
      // 1: masked tile; 2: either, decided per tile (one copy of the code)
      auto scores = [&](auto mode_c) {
        constexpr int MODE = decltype(mode_c)::value;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          if constexpr (MODE == 1) {
            mask_keys(s[kb], key0 + kb * 32 + 8 * g - key_lim);
          } else if constexpr (MODE == 2) {
            if (masked) mask_keys(s[kb], key0 + kb * 32 + 8 * g - key_lim);
            else s[kb] = f32x16_t{};
          }
#pragma unroll
          for (int kk = 0; kk < KK; ++kk) {
            const u32x4_t ak = *reinterpret_cast<const u32x4_t*>(tk + rd_off.row_off(kb, kk));
            s[kb] = (kk == 0 && MODE == 0) ? mfma32(ak, qf[kk], f32x16_t{})
                                           : mfma32(ak, qf[kk], s[kb]);
            const u32x4_t av = *reinterpret_cast<const u32x4_t*>(tv + rd_off.row_off(kb, kk));
            dp[kb] = mfma32(av, dof[kk], kk == 0 ? dp_init : dp[kb]);
          }
        }
      };
      if constexpr (D > FA2_DQ_SPLIT_MAX_D) {
        scores(std::integral_constant<int, 2>{});
      } else {
        if (masked) scores(std::integral_constant<int, 1>{});
        else scores(std::integral_constant<int, 0>{});
      }
      uint32_t dsk[KB][8];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float p0 = fast_exp2(__builtin_fmaf(s[kb][2 * i], scale_log2, -lse_q));
          const float p1 = fast_exp2(__builtin_fmaf(s[kb][2 * i + 1], scale_log2, -lse_q));
          float dp0 = dp[kb][2 * i], dp1 = dp[kb][2 * i + 1];  // dP - D if kInitD
          if constexpr (!DROP && !kInitD) {
            dp0 -= dlt;
            dp1 -= dlt;
          } else if constexpr (DROP) {
            // keys j*BC + 32kb + 16(2i/8) + 8g + (2i%8) + 0, 1: dP scaled by Z / P(keep)
            const int key = j * BC + 32 * kb + 16 * ((2 * i) / 8) + 8 * g + (2 * i) % 8;
            const uint32_t w = drop_word(drop_row, (uint32_t)key >> 1);
            dp0 = ((w << 16) >= drop.thr ? dp0 * drop.scale : 0.f) - dlt;
            dp1 = (w >= drop.thr ? dp1 * drop.scale : 0.f) - dlt;
          }
          dsk[kb][i] = pack_bf16(p0 * dp0, p1 * dp1);
        }
      if constexpr (D == 256) {
        // d = 256: each exponential between two plain VALU ops instead of runs of eight (fwd+bwd
        // step at B2 H16 N4096 +1.0-1.4%; at d = 64 and 128 within +-0.5%)
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
#pragma unroll
        for (int i = 0; i < 16 * KB; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x400, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
        }
      }
      __builtin_amdgcn_s_setprio(1);  // as in the dK/dV kernel
      // dQ^T += K^T dS^T; MFMA u covers keys 16u .. 16u+15
#pragma unroll
      for (int u = 0; u < 2 * KB; ++u) {
        const u32x4_t b = {dsk[u / 2][4 * (u % 2) + 0], dsk[u / 2][4 * (u % 2) + 1],
                           dsk[u / 2][4 * (u % 2) + 2], dsk[u / 2][4 * (u % 2) + 3]};
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          const u32x4_t a = tr_operand(tk, rd_off.tr_off(cb, u, 0), rd_off.tr_off(cb, u, 1));
          dqacc[cb] = mfma32(a, b, dqacc[cb]);
        }
      }
      __builtin_amdgcn_s_setprio(0);
    }
    FA2_STAGE_SYNC();
    wait_vmem();
    __syncthreads();
  };
  for (int j = 0; j < n_tiles; j += 2) {
    step(std::integral_constant<int, 0>{}, j);
    if (j + 1 < n_tiles) step(std::integral_constant<int, 1>{}, j + 1);
  }

  // dQ = scale * dQ_acc, queries q_wave0 .. +31 (the loop ended with a barrier: the K/V tiles
  // are free)
  static_assert(SCRATCH <= SMEM, "transpose scratch");
  store_rows_via_lds<CB, D>(smem + wave * store_scratch_bytes(CB), dqacc, scale, dq + head_off,
                            q_wave0, N, lane);
}

// ---------------------------------------------------------------------------------------
// dK, dV of grouped K/V heads whose groups were split over `split` workgroups: the sum of the
// fp32 partial sums (dK's already scaled) in split order, to bf16 in the K/V layout. 8
// elements per thread over dK (n_elem = B*Hkv*N*D elements), then dV.
template <int D>
__global__ __launch_bounds__(kThreads) void fa2_bwd_kv_reduce_kernel(
    const float* __restrict__ part, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int N,
    int n_kvheads, long long kv_bstride, int split, long long n_elem) {
  const long long e = ((long long)blockIdx.x * kThreads + threadIdx.x) * 8;
  if (e >= 2 * n_elem) return;
  const bool is_v = e >= n_elem;
  const long long ee = is_v ? e - n_elem : e;
  const float* src = part + (is_v ? (long long)split * n_elem : 0) + ee;
  f32x4_t lo = f32x4_t{}, hi = f32x4_t{};
  for (int j = 0; j < split; ++j) {
    lo += *reinterpret_cast<const f32x4_t*>(src + (long long)j * n_elem);
    hi += *reinterpret_cast<const f32x4_t*>(src + (long long)j * n_elem + 4);
  }
  const long long head_elems = (long long)N * D;
  const long long bh = ee / head_elems;  // batch * Hkv + K/V head
  const long long b = bh / n_kvheads;
  uint16_t* dst = (is_v ? dv : dk) + b * kv_bstride + (bh - b * n_kvheads) * head_elems +
                  (ee - bh * head_elems);
  *reinterpret_cast<u32x4_t*>(dst) =
      u32x4_t{pack_bf16(lo[0], lo[1]), pack_bf16(lo[2], lo[3]), pack_bf16(hi[0], hi[1]),
              pack_bf16(hi[2], hi[3])};
}

template <int D>
hipError_t launch_kv_reduce_t(const BwdArgs& a) {
  const long long n_elem = (long long)a.B * a.Hkv * a.N * D;
  const long long grid = (2 * n_elem / 8 + kThreads - 1) / kThreads;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fa2_bwd_kv_reduce_kernel<D>), dim3((unsigned)grid), dim3(kThreads), 0,
                     a.stream, a.kv_part, static_cast<uint16_t*>(a.dk),
                     static_cast<uint16_t*>(a.dv), a.N, a.Hkv, a.kv_bstride, a.kv_split, n_elem);
  return hipGetLastError();
}

hipError_t launch_kv_reduce(const BwdArgs& a) {
  if (a.d == 256) return launch_kv_reduce_t<256>(a);
  if (a.d == 64) return launch_kv_reduce_t<64>(a);
  return launch_kv_reduce_t<128>(a);
}

template <int D>
hipError_t launch_pre_t(const BwdArgs& a) {
  const long long rows = (long long)a.B * a.H * a.N;
  const long long threads = rows * (D / 8);
  const long long grid = (threads + kThreads - 1) / kThreads;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fa2_bwd_pre_kernel<D>), dim3((unsigned)grid), dim3(kThreads), 0, a.stream,
                     static_cast<const uint16_t*>(a.o), static_cast<const uint16_t*>(a.dout),
                     a.lse, a.delta, a.lse2, rows);
  return hipGetLastError();
}


template <int D, bool CAUSAL, bool DROP>
hipError_t launch_dq_t(const BwdArgs& a) {
  const int n_qblocks = (a.N + DqShape<D>::BR - 1) / DqShape<D>::BR;
  const long long grid = (long long)n_qblocks * a.B * a.H;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fa2_bwd_dq_kernel<D, CAUSAL, DROP>), dim3((unsigned)grid),
                     dim3(DqShape<D>::THREADS), 0, a.stream, static_cast<const uint16_t*>(a.q),
                     static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.v),
                     static_cast<const uint16_t*>(a.o), static_cast<const uint16_t*>(a.dout),
                     a.lse, a.lse2, a.delta, static_cast<uint16_t*>(a.dq), a.N, n_qblocks,
                     a.B * a.H, causal_window(a.B * a.H, 4ll * a.N * D, n_qblocks, D == 64 ? 2 : 1,
                                   window_budget(D)),
                     a.H, a.H / a.Hkv, a.kv_bstride, a.scale_log2, a.scale,
                     OperandSign{a.sgn_and, a.sgn_xor},
                     DropParams{a.drop_k0, a.drop_k1, a.drop_thr, a.drop_scale});
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_pre(const BwdArgs& a) {
  if (a.d == 256) return launch_pre_t<256>(a);
  return a.d == 64 ? launch_pre_t<64>(a) : launch_pre_t<128>(a);
}

template <int D, bool CAUSAL, int KP, bool DROP>
hipError_t launch_dkdv16_t(const BwdArgs& a) {
  using S = Kv16Shape<D, KP, DROP>;
  const int n_kblocks = (a.N + S::BK - 1) / S::BK;
  const long long grid = (long long)n_kblocks * a.B * a.Hkv * a.kv_split;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const int bh_count = a.B * a.Hkv * a.kv_split;
  hipLaunchKernelGGL((fa2_bwd_dkdv16_kernel<D, CAUSAL, KP, DROP>), dim3((unsigned)grid), dim3(S::THREADS),
                     0, a.stream, static_cast<const uint16_t*>(a.q),
                     static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.v),
                     static_cast<const uint16_t*>(a.dout), a.lse2, a.delta,
                     static_cast<uint16_t*>(a.dk), static_cast<uint16_t*>(a.dv), a.N, n_kblocks,
                     bh_count,
                     causal_window(bh_count, 4ll * a.N * D * (a.H / a.Hkv) / a.kv_split,
                                   n_kblocks, S::OCC, window_budget(D)),
                     a.H, a.H / a.Hkv, a.kv_bstride, a.scale_log2, a.scale,
                     OperandSign{a.sgn_and, a.sgn_xor},
                     DropParams{a.drop_k0, a.drop_k1, a.drop_thr, a.drop_scale},
                     a.kv_split > 1 ? a.kv_part : nullptr, a.kv_split);
  return hipGetLastError();
}

template <bool DROP>
hipError_t launch_bwd_dkdv_drop(const BwdArgs& a) {
  if constexpr (!DROP) {
    // 16-key MFMA blocks: at d = 256 one per wave (fwd+bwd step at B2 H16 N4096 +23-24% against
    // the 32-key kernel); at d = 64 and 128 two per wave with K in LDS and V in registers (step at
    // B4 H16 N2048 d128 +3.7% causal, +4.1% non-causal against the 32-key kernel, where one
    // sub-block per wave was 5-7.5% slower for its LDS bytes per MFMA; at B8 H32 N2048 d64 +4.2%
    // against one sub-block per wave)
    if (a.d == 256)
      return a.causal ? launch_dkdv16_t<256, true, 1, false>(a)
                      : launch_dkdv16_t<256, false, 1, false>(a);
    if (a.d == 64)
      return a.causal ? launch_dkdv16_t<64, true, 2, false>(a)
                      : launch_dkdv16_t<64, false, 2, false>(a);
    return a.causal ? launch_dkdv16_t<128, true, 2, false>(a)
                    : launch_dkdv16_t<128, false, 2, false>(a);
  } else {
    // dropout: the 16x16x32 kernel at d = 64 (dropout step at B8 H32 N2048 +8.7% causal against
    // a 32-key kernel) and, with one sub-block per wave (K and V fragments in registers, 201-202
    // VGPRs at two waves per SIMD), at d = 128 (dropout step at B4 H16 N2048 +1.5% causal, +1.2%
    // non-causal against that 32-key kernel, since removed); with two sub-blocks its dropout
    // variant spills at d = 128 and 256 (160 and ~450 bytes per lane: the keep words and -D on top
    // of 250-253 VGPRs). At d = 256 one sub-block per wave needs 370-372 VGPRs with dropout, so
    // one workgroup per CU (dropout step at B2 H16 N4096 +19% causal, +20.6% non-causal against
    // a 32-key kernel that split dK and dV over waves at two workgroups per CU, since removed)
    if (a.d == 64)
      return a.causal ? launch_dkdv16_t<64, true, 2, true>(a)
                      : launch_dkdv16_t<64, false, 2, true>(a);
    if (a.d == 256)
      return a.causal ? launch_dkdv16_t<256, true, 1, true>(a)
                      : launch_dkdv16_t<256, false, 1, true>(a);
    return a.causal ? launch_dkdv16_t<128, true, 1, true>(a)
                    : launch_dkdv16_t<128, false, 1, true>(a);
  }
}

hipError_t launch_bwd_dkdv(const BwdArgs& a) {
  const hipError_t e = a.dropout ? launch_bwd_dkdv_drop<true>(a) : launch_bwd_dkdv_drop<false>(a);
  if (e != hipSuccess || a.kv_split <= 1) return e;
  return launch_kv_reduce(a);
}

template <bool DROP>
hipError_t launch_bwd_dq_drop(const BwdArgs& a) {
  if (a.d == 256)
    return a.causal ? launch_dq_t<256, true, DROP>(a) : launch_dq_t<256, false, DROP>(a);
  if (a.d == 64) return a.causal ? launch_dq_t<64, true, DROP>(a) : launch_dq_t<64, false, DROP>(a);
  return a.causal ? launch_dq_t<128, true, DROP>(a) : launch_dq_t<128, false, DROP>(a);
}

hipError_t launch_bwd_dq(const BwdArgs& a) {
  return a.dropout ? launch_bwd_dq_drop<true>(a) : launch_bwd_dq_drop<false>(a);
}

hipError_t launch_bwd(const BwdArgs& a) {
  const hipError_t e = launch_bwd_dq(a);  // also fills the workspace (D, LSE*log2(e))
  if (e != hipSuccess) return e;
  return launch_bwd_dkdv(a);
}

// ---------------------------------------------------------------------------------------
// Backward without a caller workspace, for callers that cannot allocate device memory. The
// workspace (-D and LSE*log2(e), two fp32 [B*H*N] parts at 256-byte boundaries) lives in this
// file-scope array instead: kBwdScratchBytes on every GPU the library runs on, held from module
// load until the process ends. Each call on a GPU reuses that GPU's copy (the dQ kernel writes
// every value the dK/dV kernel reads, so nothing needs clearing), so calls that overlap on one
// GPU race.
static __device__ __align__(256) unsigned char scratch[kBwdScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};  // device address of `scratch`, per device

// The current device's copy of `scratch`: looked up once per device (with that device current)
// by hipGetSymbolAddress, since the array's name is only a host-side stand-in.
hipError_t scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}
}  // namespace

hipError_t launch_bwd_noalloc(BwdArgs a, size_t part_bytes) {
  void* base = nullptr;
  const hipError_t e = scratch_for_current_device(&base);
  if (e != hipSuccess) return e;
  a.delta = static_cast<float*>(base);
  a.lse2 = reinterpret_cast<float*>(static_cast<unsigned char*>(base) + part_bytes);
  a.kv_split = 1;
  a.kv_part = nullptr;
  return launch_bwd(a);
}

}  // namespace fa2
