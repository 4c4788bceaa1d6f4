// FlashAttention-2 forward for gfx950: O = softmax(scale Q K^T [+ causal]) V and LSE.
//
// Follows the tiled online-softmax forward (page "Flash Attention v2", "Detailed Algorithm
// Comparison / Forward Pass Comparison"; page "flashattention-2", "How FlashAttention-2
// Works (Tiled Algorithm)") with the three FlashAttention-2 changes (page "FlashAttention-2
// paper", section "Three changes"): the grid also splits the query dimension, so one head
// fills the chip; each wavefront owns 32 query rows and keeps their accumulator, running
// max and running sums in registers; the rescale by exp(m_old - m_new) is deferred until the
// running max is exceeded by more than 8 (log2 units) and the 1/l normalisation happens once
// at the end. Fully masked causal tiles are skipped (page "flashattention-2", "FlashAttention-2
// Improvements Over v1").
//
// gfx950 mapping (one workgroup = 4 waves = 128 query rows; key tiles of 64):
//  * scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: lane l owns
//    query l%32 of its wave, so row max and row sums are in-lane plus one exchange with lane
//    l^32; Q^T fragments (the B operand) stay in VGPRs for the whole key loop;
//  * O^T = V^T P^T with the same MFMA: P^T is the B operand straight from the score
//    registers (the kmap key order makes the layouts agree) and each lane's O^T column is
//    its own query, so the rescale and the final 1/l are per-lane scalars;
//  * K tiles are staged row-major and V tiles transposed (V^T) in a double-buffered LDS ring
//    with XOR-swizzled 16-byte chunks; the next tile's global loads are issued before the
//    current tile's MFMAs and written to the other LDS buffer after them (one barrier/tile);
//  * exp2 form: p = exp2(s * scale*log2(e) - m) is one FMA and one v_exp_f32; l is summed from
//    the same bf16-rounded p that feeds the MFMA (consistent convex weights), while the LSE
//    uses an fp32 sum of the unrounded p.
#include "fa2_device.hpp"
#include "fa2_launch.hpp"

namespace fa2 {

namespace {

constexpr int kFwdBR = 128;
constexpr int kFwdBC = 64;
constexpr int kFwdThreads = 256;
constexpr float kRescaleThreshold = 8.0f;  // log2 units: exponentials stay <= 2^8
constexpr float kMinusBig = -1.0e30f;      // finite start value of the running max

template <int D>
struct FwdShape {
  static constexpr int DCH = D / 8;                        // 16-byte chunks per K row
  static constexpr int KK = D / 16;                        // MFMA k-steps of the score GEMM
  static constexpr int CB = D / 32;                        // 32-row blocks of O^T
  static constexpr int K_LOADS = kFwdBC * DCH / kFwdThreads;   // 16-byte K loads per thread
  static constexpr int KPT = kFwdBC * D / 8 / kFwdThreads;     // keys per thread, V transpose
  static constexpr int KGROUPS = kFwdBC / KPT;                 // key groups per tile
  static constexpr int K_TILE_BYTES = kFwdBC * D * 2;
  static constexpr int V_TILE_BYTES = D * kFwdBC * 2;
  static constexpr int STAGE_BYTES = K_TILE_BYTES + V_TILE_BYTES;
  static_assert(K_LOADS >= 1 && KPT >= 2 && (KPT % 2) == 0, "tile shape");
  static_assert(KGROUPS * DCH == kFwdThreads, "V transpose covers the tile");
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kFwdThreads, 2) void fa2_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ o, float* __restrict__ lse,
    int N, int n_qblocks, int bh_count, float scale_log2) {
  using S = FwdShape<D>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * S::STAGE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int g = lane >> 5;

  const TileCoord tc = schedule_tile(blockIdx.x, n_qblocks, bh_count, CAUSAL);
  const size_t head_off = (size_t)tc.bh * (size_t)N * D;
  const uint16_t* qh = q + head_off;
  const uint16_t* kh = k + head_off;
  const uint16_t* vh = v + head_off;

  const int q_block0 = tc.qb * kFwdBR;
  const int q_wave0 = q_block0 + wave * 32;
  const int my_q = q_wave0 + l32;

  // ---- Q^T fragments (B operand of S^T = K Q^T): lane holds q[my_q][16kk + 8g .. +7]
  u32x4_t qf[S::KK];
  {
    const bool ok = my_q < N;
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(qh + (size_t)(ok ? my_q : 0) * D);
#pragma unroll
    for (int kk = 0; kk < S::KK; ++kk) {
      u32x4_t t = src[2 * kk + g];
      qf[kk] = ok ? t : u32x4_t{0u, 0u, 0u, 0u};
    }
  }

  // ---- number of key tiles this workgroup visits
  const int n_ktiles_all = (N + kFwdBC - 1) / kFwdBC;
  int n_ktiles = n_ktiles_all;
  if (CAUSAL) {
    const int last_key = min(N - 1, q_block0 + kFwdBR - 1);
    n_ktiles = last_key / kFwdBC + 1;
  }
  // last tile index that is not fully masked for this wave's rows
  const int wave_last_tile = CAUSAL ? min(n_ktiles - 1, (q_wave0 + 31) / kFwdBC) : n_ktiles - 1;

  // ---- global -> register staging of one K/V tile
  u32x4_t kreg[S::K_LOADS];
  u32x4_t vreg[S::KPT];
  const int vkg = tid % S::KGROUPS;  // key group (KPT keys) of this thread's V block
  const int vcc = tid / S::KGROUPS;  // 8-wide d chunk of this thread's V block

  auto load_tile = [&](int j) {
    const int key0 = j * kFwdBC;
#pragma unroll
    for (int r = 0; r < S::K_LOADS; ++r) {
      const int cid = tid + r * kFwdThreads;
      const int row = cid / S::DCH;
      const int cc = cid % S::DCH;
      const int key = key0 + row;
      u32x4_t t = {0u, 0u, 0u, 0u};
      if (key < N) t = *reinterpret_cast<const u32x4_t*>(kh + (size_t)key * D + cc * 8);
      kreg[r] = t;
    }
#pragma unroll
    for (int r = 0; r < S::KPT; ++r) {
      const int key = key0 + vkg * S::KPT + r;
      u32x4_t t = {0u, 0u, 0u, 0u};
      if (key < N) t = *reinterpret_cast<const u32x4_t*>(vh + (size_t)key * D + vcc * 8);
      vreg[r] = t;
    }
  };

  auto store_tile = [&](int stage) {
    unsigned char* sk = smem + stage * S::STAGE_BYTES;
    unsigned char* sv = sk + S::K_TILE_BYTES;
#pragma unroll
    for (int r = 0; r < S::K_LOADS; ++r) {
      const int cid = tid + r * kFwdThreads;
      const int row = cid / S::DCH;
      const int cc = cid % S::DCH;
      *reinterpret_cast<u32x4_t*>(sk + (row * S::DCH + (cc ^ kswz(row))) * 16) = kreg[r];
    }
    // transpose KPT keys x 8 d-values into 8 rows of V^T, KPT keys each
    const int chunk = (vkg * S::KPT) / 8;
    const int sub = ((vkg * S::KPT) % 8) * 2;  // byte offset inside the 16-byte chunk
#pragma unroll
    for (int e = 0; e < 4; ++e) {      // dword e of the 8-wide chunk: d = 8*vcc + 2e, +1
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int c = vcc * 8 + 2 * e + half;
        uint32_t w[S::KPT / 2];
#pragma unroll
        for (int p = 0; p < S::KPT / 2; ++p) {
          const uint32_t a = vreg[2 * p][e], b = vreg[2 * p + 1][e];
          w[p] = half ? __builtin_amdgcn_perm(b, a, 0x07060302u)
                      : __builtin_amdgcn_perm(b, a, 0x05040100u);
        }
        unsigned char* dst = sv + (c * 8 + (chunk ^ vswz(c))) * 16 + sub;
        if constexpr (S::KPT == 4) {
          *reinterpret_cast<u32x2_t*>(dst) = u32x2_t{w[0], w[1]};
        } else {
          *reinterpret_cast<uint32_t*>(dst) = w[0];
        }
      }
    }
  };

  // ---- per-lane LDS read offsets (bytes, within a stage). The swizzle only touches the low 3
  // bits of the chunk index and does not depend on row bits >= 4, so block kb, k-step group
  // kk/4 and d-block pair cb/2 become immediate offsets on a few base registers.
  const int krow = kmap(l32);
  int koff[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) koff[kk] = (krow * S::DCH + ((2 * kk + g) ^ kswz(krow))) * 16;
  auto k_off = [&](int kb, int kk) {
    return koff[kk & 3] + (kk >> 2) * 128 + kb * 32 * S::DCH * 16;
  };
  int voff[2][4];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int c = cb * 32 + l32;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      voff[cb][u] = S::K_TILE_BYTES + (c * 8 + ((2 * u + g) ^ vswz(c))) * 16;
  }
  auto v_off = [&](int cb, int u) { return voff[cb & 1][u] + (cb >> 1) * 64 * 8 * 16; };

  // ---- accumulators and row statistics (per lane: query my_q, half g of the keys)
  f32x16_t oacc[S::CB];
#pragma unroll
  for (int cb = 0; cb < S::CB; ++cb) oacc[cb] = f32x16_t{};
  float m_run = kMinusBig;  // running max of scale*log2(e)*s (possibly stale by < threshold)
  float l_f32 = 0.f;        // partial sum of p over this lane's keys (fp32, for LSE)
  float l_bf = 0.f;         // partial sum of bf16(p) (normaliser of O)

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int j = 0; j < n_ktiles; ++j) {
    const int stage = j & 1;
    if (j + 1 < n_ktiles) load_tile(j + 1);

    if (j <= wave_last_tile) {
      const unsigned char* sbase = smem + stage * S::STAGE_BYTES;
      // S^T tile: two 32-key blocks x 32 queries
      f32x16_t s[2] = {f32x16_t{}, f32x16_t{}};
#pragma unroll
      for (int kk = 0; kk < S::KK; ++kk) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const u32x4_t a = *reinterpret_cast<const u32x4_t*>(sbase + k_off(kb, kk));
          s[kb] = mfma32(a, qf[kk], s[kb]);
        }
      }

      // masking: key index of register i of block kb is key0 + 32kb + 16(i/8) + 8g + i%8
      const int key0 = j * kFwdBC;
      const bool need_mask = (key0 + kFwdBC > N) || (CAUSAL && key0 + kFwdBC - 1 > q_wave0);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = key0 + kb * 32 + (i / 8) * 16 + g * 8 + (i % 8);
            const bool masked = (key >= N) || (CAUSAL && key > my_q);
            s[kb][i] = masked ? -INFINITY : s[kb][i];
          }
      }

      // online softmax, exp2 form, deferred rescale
      float mx = s[0][0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[0][i]);
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[1][i]);
      mx = max_xor32(mx);
      const float m_tile = mx * scale_log2;
      const bool raise = m_tile > m_run + kRescaleThreshold;
      if (__builtin_amdgcn_ballot_w64(raise) != 0) {
        const float m_new = fmaxf(m_run, m_tile);
        const float alpha = fast_exp2(m_run - m_new);
        m_run = m_new;
        l_f32 *= alpha;
        l_bf *= alpha;
#pragma unroll
        for (int cb = 0; cb < S::CB; ++cb) oacc[cb] *= alpha;
      }
      const float neg_m = -m_run;
      uint32_t pk[2][8];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float p0 = fast_exp2(__builtin_fmaf(s[kb][2 * i], scale_log2, neg_m));
          const float p1 = fast_exp2(__builtin_fmaf(s[kb][2 * i + 1], scale_log2, neg_m));
          l_f32 += p0 + p1;
          const uint32_t w = pack_bf16(p0, p1);
          pk[kb][i] = w;
          l_bf = add_bf16_pair(l_bf, w);
        }

      // O^T += V^T P^T: MFMA u covers keys 16u .. 16u+15, i.e. score block u/2, regs 8(u%2)..
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const u32x4_t b = {pk[u / 2][4 * (u % 2) + 0], pk[u / 2][4 * (u % 2) + 1],
                           pk[u / 2][4 * (u % 2) + 2], pk[u / 2][4 * (u % 2) + 3]};
#pragma unroll
        for (int cb = 0; cb < S::CB; ++cb) {
          const u32x4_t a = *reinterpret_cast<const u32x4_t*>(sbase + v_off(cb, u));
          oacc[cb] = mfma32(a, b, oacc[cb]);
        }
      }
    }

    if (j + 1 < n_ktiles) store_tile(stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue: deferred normalisation, bf16 output, LSE
  const float l_tot = sum_xor32(l_f32);
  const float lb_tot = sum_xor32(l_bf);
  if (my_q < N) {
    const float inv = fast_rcp(lb_tot);
    uint16_t* orow = o + head_off + (size_t)my_q * D;
#pragma unroll
    for (int cb = 0; cb < S::CB; ++cb)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int c = cb * 32 + 8 * t + 4 * g;
        u32x2_t w = {pack_bf16(oacc[cb][4 * t + 0] * inv, oacc[cb][4 * t + 1] * inv),
                     pack_bf16(oacc[cb][4 * t + 2] * inv, oacc[cb][4 * t + 3] * inv)};
        *reinterpret_cast<u32x2_t*>(orow + c) = w;
      }
    if (g == 0) lse[(size_t)tc.bh * N + my_q] = (m_run + fast_log2(l_tot)) * kLn2;
  }
}

template <int D, bool CAUSAL>
hipError_t launch_fwd_t(const FwdArgs& a) {
  const int n_qblocks = (a.N + kFwdBR - 1) / kFwdBR;
  const long long grid = (long long)n_qblocks * a.B * a.H;
  if (grid <= 0 || grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fa2_fwd_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(kFwdThreads), 0,
                     a.stream, static_cast<const uint16_t*>(a.q),
                     static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.v),
                     static_cast<uint16_t*>(a.o), a.lse, a.N, n_qblocks, a.B * a.H,
                     a.scale_log2);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a) {
  if (a.d == 64) return a.causal ? launch_fwd_t<64, true>(a) : launch_fwd_t<64, false>(a);
  return a.causal ? launch_fwd_t<128, true>(a) : launch_fwd_t<128, false>(a);
}

}  // namespace fa2
