// Device-side building blocks shared by the gfx950 attention kernels: vector types, the
// bf16 MFMA wrapper, bf16 packing, cross-half lane exchange, LDS swizzles and the
// workgroup -> (query block, batch*head) schedule.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa2 {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

#define FA2_LDS __attribute__((address_space(3)))

// Buffer resource over [base, base + bytes): loads beyond `bytes` return zeros, which is how
// ragged sequence tails are padded without branches. (Word 3 = 0x00020000 selects the plain
// 32-bit data format on gfx9-family parts.)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// 16-byte buffer load into registers (zeros when out of range).
__device__ __forceinline__ u32x4_t buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                 uint32_t soff) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// 16 bytes per lane from global memory straight into LDS (no VGPRs): lane l's data lands at
// lds_wave_base + 16*l; lds_wave_base must be wave-uniform. Zeros when out of range.
__device__ __forceinline__ void buffer_load16_to_lds(__amdgpu_buffer_rsrc_t r,
                                                     void* lds_wave_base, uint32_t voff,
                                                     uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (FA2_LDS void*)lds_wave_base, 16, voff, soff, 0, 0);
}

// Transposing LDS read of 16-bit data (ds_read_b64_tr_b16). Within each group of 16 lanes,
// lane i receives element (i % 4) of the 8-byte chunks addressed by lanes i/4, i/4 + 4,
// i/4 + 8 and i/4 + 12 (in that order). If lane j of the group addresses row r0 + j/4,
// columns c0 + 4*(j%4) .. +3 of a row-major bf16 matrix, lane i receives column c0 + i of
// rows r0 .. r0+3: a column slice, i.e. the transposed operand an MFMA needs.
__device__ __forceinline__ u32x2_t lds_read_tr16(const void* p) {
  s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA2_LDS s16x4_t*)(p));
  return __builtin_bit_cast(u32x2_t, v);
}

// Wait until this wave's outstanding vector-memory loads (including loads into LDS) are done.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Extra synchronisation for race checks (builds with -DFA2_DEBUG_SYNC): at every hand-over of an
// LDS stage, each wave waits for all of its outstanding loads and the workgroup meets at a
// barrier, so no tile is read before every wave's loads into it have landed and no stage is
// refilled while a wave may still read it, whatever the normal build's waits allow. Results
// must not change by a single bit; the normal build compiles this away.
#ifdef FA2_DEBUG_SYNC
#define FA2_STAGE_SYNC()  \
  do {                    \
    wait_vmem();          \
    __syncthreads();      \
  } while (0)
#else
#define FA2_STAGE_SYNC() \
  do {                   \
  } while (0)
#endif

constexpr float kLn2 = 0.69314718055994530942f;

// D(32x32) += A(32x16) * B(16x32), bf16 inputs, fp32 accumulate (v_mfma_f32_32x32x16_bf16).
// Lane l holds A[l%32][8*(l/32) + i] and B[8*(l/32) + i][l%32] for i = 0..7; the result
// register i of lane l is D[8*(i/4) + 4*(l/32) + (i%4)][l%32].
__device__ __forceinline__ f32x16_t mfma32(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Two fp32 values -> one dword of two bf16 (round to nearest even, v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// acc + lo(w) + hi(w), the two bf16 halves of w widened exactly (v_dot2c_f32_bf16 with 1.0).
__device__ __forceinline__ float add_bf16_pair(float acc, uint32_t w) {
  const bf16x2_t one = __builtin_bit_cast(bf16x2_t, 0x3F803F80u);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), one, acc, false);
}

// max / sum of x over lanes l and l^32 (the two halves of a wave hold the two halves of
// one query's key set). v_permlane32_swap exchanges the upper half of its first operand
// with the lower half of its second; applied to (x, x) the two results hold x[l] and
// x[l^32] in some order in every lane, so a commutative combine needs no lane select.
__device__ __forceinline__ float max_xor32(float x) {
  int xi = __float_as_int(x);
  auto r = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
  return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  int xi = __float_as_int(x);
  auto r = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// Key order inside a 32-key MFMA block: M-row m of the score MFMA reads key kmap(m), which
// swaps bits 2 and 3 of m. With this order lane l's 16 score registers hold keys
// 8*(l/32) + 0..7 (registers 0..7) and 16 + 8*(l/32) + 0..7 (registers 8..15), exactly
// the B-operand layout the P*V MFMA needs, so P never leaves registers.
__device__ __forceinline__ int kmap(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// XOR swizzle of the 16-byte chunks of a row-major bf16 tile with D columns: physical chunk =
// logical chunk ^ swz<D>(row). gfx950's LDS has 64 banks of 4 bytes (256 bytes per cycle); a
// ds_read_b128 serves 16 lanes per cycle and a ds_read_b64_tr_b16 32 lanes. The two read
// patterns of the kernels are
//   (a) MFMA operand rows: 16 lanes read one logical chunk of 16 different rows (any 16
//       consecutive rows, possibly permuted by kmap);
//   (b) transposing reads: 32 lanes read rows 4a .. 4a+3, four adjacent chunks per row.
// For D = 128 a row is the whole 256-byte bank window: (a) needs swz injective on 16 rows, (b)
// needs bits 2-3 of swz to differ across rows 4a .. 4a+3; ((row & 3) << 2) | ((row >> 2) & 3)
// does both. For D = 256 a row spans two windows and every row starts on a window boundary,
// so the bank of a chunk depends on its index mod 16 only: the D = 128 swizzle applies to chunk
// bits 0-3 (chunk bit 4 is unchanged). For D = 64 two rows share the window (row parity picks
// the half), so swz must be injective on rows of one parity for (a) and differ in bit 2
// between rows 4a and 4a+2 (and 4a+1, 4a+3) for (b): (bit 1 of row) << 2 | ((row >> 2) & 3).
template <int D>
__device__ __forceinline__ int swz(int row) {
  static_assert(D == 64 || D == 128 || D == 256, "head dimension");
  if constexpr (D >= 128) return ((row & 3) << 2) | ((row >> 2) & 3);
  return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

// The sign of the softmax scale, carried by one operand of the score product. The kernels form
// scores as c * (q . k) with c > 0 (the running max and the -inf mask start rely on it); a
// scale < 0 is applied as c = |scale| with one operand's bf16 sign bits flipped (flipping is
// exact, and (-q) . k = -(q . k) wherever the accumulation rounds symmetrically in sign, as
// round-to-nearest does), and scale = 0 as that operand zeroed (every score exactly 0, any
// c > 0). x -> (x & and_mask) ^ xor_mask on each dword: (~0, 0) keeps the operand,
// (~0, 0x80008000) negates it, (0, 0) zeroes it.
struct OperandSign {
  uint32_t and_mask, xor_mask;
};
__device__ __forceinline__ u32x4_t apply_sign(u32x4_t x, const OperandSign& sg) {
  return (x & sg.and_mask) ^ sg.xor_mask;
}

// XOR swizzle of the query tiles of the 16-key dK/dV kernel, whose read patterns differ from the
// ones above: (a) MFMA operand rows: lane l reads logical chunk 4k + l/16 of row l%16; (b)
// transposing reads: lanes 0-31 (then 32-63) read rows 8a .. 8a+7, an even chunk and the next in
// each. gfx950's LDS, as measured by counter probes (two active lanes at a time, the bank-
// conflict counter per pair): 64 banks of 4 bytes; a ds_read_b64 serves lanes 0-31, then
// 32-63; a ds_read_b128 serves 16 lanes per cycle, lanes 0-3, 12-15, 20-27 together (the
// 4-lane quads of a half-wave grouped by the parity of lane bits 2-4), then the other quads,
// then the same for lanes 32-63. With row = l%16 in (a), one such group reads rows 0-3 and
// 12-15 at chunk group g and rows 4-11 at g + 1, so swz must map rows 4-11 onto a set closed
// under XOR 1 (the chunk-group step), and (b) needs swz bits 1-3 to differ across 8 aligned
// rows. For D >= 128 (a row fills the 256-byte bank window; at D = 256 chunk bit 4 stays)
// swz = (row & 7) << 1 does both; for D = 64 (two rows per window, the row parity picks the
// half) swz = ((row >> 1) & 3) << 1. A swizzle bijective on 16 rows, (row & 7) << 1 | bit 3 of
// row, measured 2-way conflicts on (a): 8 cycles and 4 conflict cycles per instruction.
template <int D>
__device__ __forceinline__ int swz16(int row) {
  static_assert(D == 64 || D == 128 || D == 256, "head dimension");
  if constexpr (D >= 128) return (row & 7) << 1;
  return ((row >> 1) & 3) << 1;
}

// D(16x16) += A(16x32) * B(32x16), bf16 inputs, fp32 accumulate (v_mfma_f32_16x16x32_bf16).
// Lane l holds A[l%16][8*(l/16) + i] and B[8*(l/16) + i][l%16] for i = 0..7; the result
// register r of lane l is D[4*(l/16) + r][l%16] (layout checked on gfx950 against a CPU product).
__device__ __forceinline__ f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Dropout mask generator: the 32-bit PCG-based hash of Jarzynski and Olano ("Hash Functions for
// GPU Rendering", JCGT 9(3), 2020), an LCG step followed by a random xorshift, a multiply and
// a fixed xorshift. For query head bh: a = hash(k0 ^ hash(k1 ^ bh)) (k0, k1 from the seed and
// offset), row key r_i = hash(a ^ i), and one word w = hash(r_i ^ m*0x9E3779B9) per key pair
// m = j/2: key 2m is kept iff the low 16 bits of w are >= t, key 2m+1 iff the high 16 bits
// are, t = floor(p * 2^16). The kernels compare whole words against thr = t << 16: the high
// half as w >= thr, the low half as (w << 16) >= thr.
__device__ __forceinline__ uint32_t pcg_hash(uint32_t x) {
  const uint32_t state = x * 747796405u + 2891336453u;
  const uint32_t word = ((state >> ((state >> 28u) + 4u)) ^ state) * 277803737u;
  return (word >> 22u) ^ word;
}
constexpr uint32_t kDropKeyMul = 0x9E3779B9u;
struct DropParams {
  uint32_t k0, k1;  // seed and offset keys
  uint32_t thr;     // t << 16: keep iff the key's 16 bits, moved to the top, are >= thr
  float scale;      // 1 / P(keep)
};
__device__ __forceinline__ uint32_t drop_head_key(const DropParams& dp, uint32_t bh) {
  return pcg_hash(dp.k0 ^ pcg_hash(dp.k1 ^ bh));
}
// The word of row key r and key pair m.
__device__ __forceinline__ uint32_t drop_word(uint32_t r, uint32_t m) {
  return pcg_hash(r ^ (m * kDropKeyMul));
}
// The value of the neighbouring lane (lane ^ 1), by DPP quad_perm [1, 0, 3, 2].
__device__ __forceinline__ uint32_t swap_adjacent_lanes(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false);
}

// Stores a wave's 32-row tile of results, NB column blocks of 32 held as MFMA results (lane l:
// row l % 32; register 4t + e of block cb: column 32cb + 8t + 4(l/32) + e), times `mul` (per
// lane, i.e. per row), as bf16 into rows row0 .. row0+31 of `out` (row stride LD elements, `out`
// at the tile's first column; rows >= n_rows are skipped). Up to 128 columns at a time go
// through `scratch` (LDS that only this wave uses, store_scratch_bytes(NB) bytes, rows padded
// by 16 bytes), so that each global store writes whole row segments, 16 bytes per lane, rather
// than 8 bytes in each of 32 rows.
constexpr int store_scratch_bytes(int nb) { return 32 * (64 * (nb < 4 ? nb : 4) + 16); }
template <int NB, int LD>
__device__ __forceinline__ void store_rows_via_lds(unsigned char* scratch, const f32x16_t* acc,
                                                   float mul, uint16_t* out, int row0,
                                                   int n_rows, int lane) {
  constexpr int W = NB < 4 ? NB : 4;        // column blocks per pass
  constexpr int PITCH = 64 * W + 16;
  constexpr int CH = 4 * W, RPI = 64 / CH;  // 16-byte chunks per row, rows per store
  const int r = lane & 31, g = lane >> 5;
#pragma unroll
  for (int c0 = 0; c0 < NB; c0 += W) {
#pragma unroll
    for (int cb = 0; cb < W; ++cb)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        *reinterpret_cast<u32x2_t*>(scratch + r * PITCH + (32 * cb + 8 * t + 4 * g) * 2) =
            u32x2_t{pack_bf16(acc[c0 + cb][4 * t] * mul, acc[c0 + cb][4 * t + 1] * mul),
                    pack_bf16(acc[c0 + cb][4 * t + 2] * mul, acc[c0 + cb][4 * t + 3] * mul)};
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int rr = i * RPI + lane / CH, ch = lane % CH;
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(scratch + rr * PITCH + ch * 16);
      if (row0 + rr < n_rows)
        *reinterpret_cast<u32x4_t*>(out + (size_t)(row0 + rr) * LD + 32 * c0 + ch * 8) = v;
    }
  }
}

// Accumulator start values of a masked 32x32 score block: -inf for hidden entries, 0 otherwise.
// Lane = query, registers = keys (the forward and dQ layout): register i holds key
// base + 16(i/8) + 8g + i%8; mask_keys takes rel = (key of register 0) - key_lim, the lane's
// key_lim being the last visible key (min(query, N - 1) causal, N - 1 otherwise), so register i
// is hidden iff rel + 16(i/8) + i%8 > 0: one compare against a constant per register.
__device__ __forceinline__ void mask_keys(f32x16_t& s, int rel) {
#pragma unroll
  for (int i = 0; i < 16; ++i) s[i] = rel > -(16 * (i / 8) + (i % 8)) ? -INFINITY : 0.f;
}
// Workgroup id -> (block, batch*head) order. Workgroups are dealt to the 8 XCDs in turn
// (id % 8), each XCD with its own L2; when the heads divide evenly, XCD x gets the heads
// x, x+8, ... only.
//  * kHeadMajor (equal-length blocks, no mask): an XCD runs one head's blocks back to back,
//    so that head's K/V tiles are re-read from its L2.
//  * kLongDescending / kLongAscending (causal: block lengths differ): an XCD takes its heads in
//    windows of `window` heads and deals each window's blocks longest first (rank-major over
//    the window's heads: a list schedule in longest-processing-time order, so no long block
//    starts near the end of the window), one window after the other. The window is as many
//    heads as a budget of L2 bytes holds the streamed tiles of (at least enough blocks to fill
//    the XCD), so the blocks in flight walk the tiles of fewer heads. At d = 64 (three forward
//    workgroups per CU, 96 blocks of 32 heads in flight) dealing all heads at once moved 3.8x
//    the compulsory bytes and bound the forward on memory; windows of 16 heads cut that and ran
//    the forward 6.6% faster. At d >= 128 the kernels are not bound by these refetches and
//    smaller windows measured neutral to 3% slower, so the window is all of the XCD's heads.
//    Descending: the highest block index is the longest (query blocks of the forward and dQ);
//    ascending: the lowest is (key blocks of dK/dV).
enum class Order { kHeadMajor, kLongDescending, kLongAscending };
struct TileCoord {
  int qb;
  int bh;
};
template <Order O>
__device__ __forceinline__ TileCoord schedule_tile(int wg, int n_blocks, int bh_count,
                                                   int window) {
  int r, bh;
  if ((bh_count & 7) == 0) {
    const int xcd = wg & 7;
    const int j = wg >> 3;
    if constexpr (O == Order::kHeadMajor) {
      bh = (j / n_blocks) * 8 + xcd;
      r = j % n_blocks;
    } else {
      const int hpx = bh_count >> 3;
      if (window >= hpx) {  // one window: rank-major over all of the XCD's heads
        bh = (j % hpx) * 8 + xcd;
        r = j / hpx;
      } else {
        const int per_window = window * n_blocks;
        const int w = j / per_window;
        const int in = j - w * per_window;
        const int wh = min(window, hpx - w * window);  // heads in this (possibly last) window
        bh = (w * window + in % wh) * 8 + xcd;
        r = in / wh;
      }
    }
  } else {
    bh = wg % bh_count;
    r = wg / bh_count;
  }
  TileCoord t;
  t.qb = O == Order::kLongDescending ? (n_blocks - 1 - r) : r;
  t.bh = bh;
  return t;
}

}  // namespace fa2
