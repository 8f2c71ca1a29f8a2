// The trellis linear with the row-by-weight products on the matrix cores.
//
// Same projection, stream format, decode and finish as the v_dot2 linear
// (TensorFold pull request "hip exl3: the input rotation and trellis linear for
// decode rows", "What this changes"); only the sums over k move from
// v_dot2_f32_f16 chains to v_mfma_f32_16x16x32_f16, so the vector ALUs spend
// their cycles on decoding and the time grows slowly with the number of rows.
//
// One workgroup per (128-column strip, pass of up to 16 rows). A wave step
// covers a pair of tile rows, k = 32p .. 32p + 31 (wave w takes p = w, w +
// WAVES, ...), and runs eight MFMAs, one per 16-column tile m of the strip:
//  - B (32 k x 16 n): lane l = 16g + n holds B[8g + t][n] = W[32p + 8g + t]
//    [128 strip + 16m + n], t = 0..7: k-group g is tile row 2p + (g >> 1),
//    k-half g & 1, of column n of tile m. These 8 values are 8 consecutive
//    windows of the tile (value index 16n + 8(g & 1) + t). The wave brings
//    each tile row in with one coalesced load (as the v_dot2 linear does) and
//    writes it to a wave-private LDS stage one step ahead; the lane reads back
//    the 2 or 3 dwords that hold its k-half's 7*BITS + 16 bits (wrapping inside
//    the tile), realigns them when the k-half does not start on a dword, and
//    decodes its B operand directly: no lane exchange, no zero padding;
//  - A (16 rows x 32 k): lane 16g + r holds z[r][32p + 8g .. 32p + 8g + 7],
//    one 16-byte load per lane per step (rows past the pass repeat its last
//    row and are never stored);
//  - D: lane 16g + n holds D[4g + i][n], i = 0..3: pass row 4g + i, strip
//    column 16m + n.
// A row's D entries depend only on its own A row, and every pass, whatever its
// row count, runs the same instruction over the same k groups in the same
// order (pairs ascending per wave, then the waves' sums in wave order), so a
// row's bits never depend on the rows that share its launch. The order is a
// different fixed one from the v_dot2 linear's: the two agree to the float64
// gate, not bit for bit. Narrow matrices at 4 waves run a column-split form
// with the same bits (see linear_mfma_kernel's PARTS).
#include "exl3_launch.hpp"
#include "exl3_strip.hpp"

namespace tf_exl3 {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ half8_t pairs_to_half8(half2_t a, half2_t b, half2_t c, half2_t d) {
  uint4 u;
  u.x = __builtin_bit_cast(uint32_t, a);
  u.y = __builtin_bit_cast(uint32_t, b);
  u.z = __builtin_bit_cast(uint32_t, c);
  u.w = __builtin_bit_cast(uint32_t, d);
  return __builtin_bit_cast(half8_t, u);
}

// Dwords a lane loads for one k-half: its windows span 7*BITS + 16 bits and
// start at bit (16n + 8h)*BITS of the tile, up to 24 bits into a dword.
template <int BITS>
constexpr int khalf_raw_words() {
  return BITS <= 4 ? 2 : 3;
}

// Realigned dwords (bit 0 = the first window's bit 0) that hold the 8 windows.
template <int BITS>
constexpr int khalf_words() {
  return (7 * BITS + 16 + 31) / 32;
}

// Whether every k-half starts on a dword boundary (4 and 8 bits), so no
// realignment is needed.
template <int BITS>
constexpr bool khalf_aligned() {
  return (8 * BITS) % 32 == 0;
}

// The 8 states of a k-half from its realigned dwords a[] (window j at bit
// j*BITS; a[khalf_words] is zero). When BITS divides 16 and the window 16 bits
// on is in the same k-half, one funnel shift gives both (as in lane_states).
template <int BITS, int I = 0>
__device__ __forceinline__ void khalf_states(const uint32_t (&a)[khalf_words<BITS>() + 1], uint32_t (&st)[8]) {
  if constexpr (I < 8) {
    constexpr int o = I * BITS;
    constexpr int d = o >> 5;
    constexpr int sh = o & 31;
    if constexpr (16 % BITS == 0 && 16 / BITS < 8) {
      if constexpr (sh < 16) {
        uint32_t t;
        if constexpr (sh == 0) {
          t = a[d];
        } else {
          t = funnel<sh>(a[d + 1], a[d]);
        }
        st[I] = t & 0xFFFFu;
        if constexpr (I + 16 / BITS < 8) st[I + 16 / BITS] = t >> 16;
      }
    } else {
      st[I] = window_at<BITS>(a, I);
    }
    khalf_states<BITS, I + 1>(a, st);
  }
}

// LDS stage of one pair's stream for one wave: two tile rows of the wave's
// tiles (all 8, or 8 / PARTS in the column-split forms), the second padded to
// start 32 banks (mod 64) after the first, so the two halves of the wave, which
// read different tile rows, read different banks.
template <int BITS, int PARTS>
constexpr int stage_row_words() {
  return 64 * BITS / PARTS + (96 - (64 * BITS / PARTS) % 64) % 64;
}
template <int BITS, int PARTS>
constexpr int stage_words() {
  return 2 * stage_row_words<BITS, PARTS>();
}

// Lanes that load a tile row of the wave's tiles (WORDS dwords): 64, or 32 where
// 64 does not divide it (the split form at odd widths); lanes past them repeat
// their words (the same line, coalesced) and write the same values to the same
// stage words.
template <int WORDS>
constexpr int load_lanes() {
  return WORDS % 64 == 0 ? 64 : 32;
}
constexpr int kWaveLdsWords = kRowsPerPass * kBlock;  // one k-wave's partial sums, 8 KiB

// PARTS = 1: WAVES waves, each decodes all 8 tiles of its pairs; its stage
// lives in its own partial-sum area. PARTS = 2 (column split, for narrow
// launches): 2 * WAVES waves, wave (h, w) takes the same pairs as wave w of the
// first form but only tiles 4h .. 4h + 3 (NT = 8 / PARTS), so each column sees
// the same MFMAs in the same order and the same cross-wave sum: the outputs are
// bit-identical to the first form's. (Quarters over four times the waves were
// measured too: no faster at one row, slower at 16, where every extra wave
// loads its own A operand.)
template <int BITS, int WAVES, int PARTS>
__global__ __launch_bounds__(kWave* WAVES* PARTS) __attribute__((amdgpu_waves_per_eu(4))) void linear_mfma_kernel(
    const uint16_t* __restrict__ z, const uint32_t* __restrict__ trellis, const uint16_t* __restrict__ svh,
    void* __restrict__ y, int y_dtype, int rows, int in_dim, int out_dim) {
  constexpr int NR = kRowsPerPass;
  constexpr int NT = 8 / PARTS;  // tiles (MFMAs) per wave and pair
  constexpr int CW = khalf_raw_words<BITS>();
  constexpr int KW = khalf_words<BITS>();
  // Pairs in flight. The stage takes step i + 1's stream during step i, so PF
  // pairs in flight give PF - 1 steps of cover: at least 2, except the 8-bit
  // first form, where a second pair spills past 128 VGPRs (measured on the 8-bit
  // LM head at 16 rows: 145 us against 140 with one pair; its many waves cover).
  // The column-split form runs narrow launches at about two waves per SIMD, so
  // each wave keeps twice the pairs in flight (a pair is half the first form's
  // bytes there).
  constexpr int PF_WIDE = prefetch_depth<BITS>() / 2 > 2 ? prefetch_depth<BITS>() / 2 : 2;
  constexpr int PF = PARTS >= 2 ? 2 * PF_WIDE : BITS == 8 ? 1 : PF_WIDE;
  constexpr int RING = PF + 1;
  constexpr int RS = stage_row_words<BITS, PARTS>();  // stage words from tile row 2p to 2p + 1
  // Loads of a tile row's NT tiles (8 * BITS * NT words): LW lanes take PW contiguous dwords each.
  constexpr int LW = load_lanes<8 * BITS * NT>();
  constexpr int PW = 8 * BITS * NT / LW;
  static_assert(LW * PW == 8 * BITS * NT, "the wave's loads cover its tiles");
  static_assert(PARTS == 1 ? stage_words<BITS, 1>() <= kWaveLdsWords : true, "the stage fits the partial area");
  constexpr int LDS_WORDS = PARTS == 1 ? WAVES * kWaveLdsWords
                                       : WAVES * kWaveLdsWords + WAVES * PARTS * stage_words<BITS, PARTS>();
  __shared__ __attribute__((aligned(16))) uint32_t lds[LDS_WORDS];

  const int lane = __lane_id();
  const int hw = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = hw / WAVES;
  const int wave = hw - half * WAVES;  // the k split, as in the first form
  const int strip = blockIdx.x;
  const int r0 = blockIdx.y * NR;
  const int nr = min(NR, rows - r0);
  const int pairs = in_dim / 32;
  const int iters = (pairs - wave + WAVES - 1) / WAVES;  // 0 when in_dim = 128 and WAVES = 8, wave >= 4
  uint32_t* const stage = PARTS == 1 ? lds + wave * kWaveLdsWords
                                     : lds + WAVES * kWaveLdsWords + hw * stage_words<BITS, PARTS>();

  // Stream walk: tile rows 2p and 2p + 1 of the wave's pair p, its NT tiles of
  // each (one coalesced load per tile row; in the split forms, where a tile row of
  // NT tiles is fewer than 64 lanes' dwords, lanes past LW repeat a lower lane's
  // words, which they write to the same place).
  const StreamStrides st = stream_strides<BITS>(kLayoutTiles, in_dim, out_dim);
  const uint32_t* __restrict__ tbase = trellis + (size_t)strip * st.strip + half * NT * 8 * BITS;
  const int off = (lane % LW) * PW;
  auto pair_ptr = [&](int i) { return tbase + (size_t)(2 * min(wave + i * WAVES, pairs - 1)) * st.row; };
  // A operand: lane 16g + r holds z[r][32p + 8g .. + 7] (rows past the pass repeat its last row).
  const int g = lane >> 4;
  const int n = lane & 15;
  const uint4* __restrict__ zsrc =
      reinterpret_cast<const uint4*>(z + (size_t)(r0 + min(n, nr - 1)) * in_dim + 8 * g);
  auto zload = [&](int i) { return zsrc[(size_t)min(wave + i * WAVES, pairs - 1) * 4]; };

  // B operand: lane 16g + n decodes k-half g & 1 of column n of each of the
  // wave's tiles in tile row 2p + (g >> 1); its dwords sit at these stage
  // offsets (tile m adds 8*BITS*m).
  const int bit0 = (16 * n + 8 * (g & 1)) * BITS;
  const int sh = bit0 & 31;
  int roff[CW];
#pragma unroll
  for (int c = 0; c < CW; ++c) roff[c] = (g >> 1) * RS + ((bit0 >> 5) + c) % (8 * BITS);

  uint32_t ring[RING][2][PW];
  uint4 zr[RING];
  auto issue = [&](uint32_t (&dst)[2][PW], uint4& zd, int i) __attribute__((always_inline)) {
    zd = zload(i);
    const uint32_t* p = pair_ptr(i);
    load_share<PW>(dst[0], p, off);
    load_share<PW>(dst[1], p + st.row, off);
  };
  auto put = [&](const uint32_t (&src)[2][PW]) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int c = 0; c < PW; ++c) stage[t * RS + off + c] = src[t][c];
    }
  };

  f32x4 acc[NT];
#pragma unroll
  for (int m = 0; m < NT; ++m) acc[m] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

#pragma unroll
  for (int d = 0; d < PF; ++d) issue(ring[d], zr[d], d);
  put(ring[0]);

  // Step i: loads for step i + PF; this step's dwords out of the stage; step
  // i + 1's stream into the stage (LDS runs a wave's accesses in order, so the
  // reads above see step i); decode and the MFMAs.
  auto step = [&](auto dc, int i) __attribute__((always_inline)) {
    constexpr int D = decltype(dc)::value;
    issue(ring[(D + PF) % RING], zr[(D + PF) % RING], i + PF);
    // In the split forms (registers to spare) this keeps the loads at the top of
    // the step: left to itself the scheduler sank them below the decode at 3
    // bits, and the next step's stage write then waited for loads just issued.
    // The first form keeps the scheduler's order: there the pin costs spills.
    if constexpr (PARTS >= 2) asm volatile("" ::: "memory");
    uint32_t kh[NT][CW];
#pragma unroll
    for (int m = 0; m < NT; ++m) {
#pragma unroll
      for (int c = 0; c < CW; ++c) kh[m][c] = stage[roff[c] + m * 8 * BITS];
    }
    put(ring[(D + 1) % RING]);
    const half8_t a = __builtin_bit_cast(half8_t, zr[D]);
#pragma unroll
    for (int m = 0; m < NT; ++m) {
      uint32_t al[KW + 1];
#pragma unroll
      for (int c = 0; c < KW; ++c) {
        if constexpr (khalf_aligned<BITS>()) {
          al[c] = kh[m][c];
        } else {
          al[c] = __builtin_amdgcn_alignbit(c + 1 < CW ? kh[m][c + 1] : 0u, kh[m][c], sh);
        }
      }
      al[KW] = 0u;
      uint32_t s8[8];
      khalf_states<BITS>(al, s8);
      const half8_t b = pairs_to_half8(decode_pair(s8[0], s8[1]), decode_pair(s8[2], s8[3]),
                                       decode_pair(s8[4], s8[5]), decode_pair(s8[6], s8[7]));
      acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[m], 0, 0, 0);
    }
  };
  step_loop<RING>(iters, step);

  // D entry i of acc[m]: pass row 4g + i, strip column 16 (NT half + m) + n, into
  // k-wave `wave`'s partial sums (in the first form that area held the wave's
  // stage, whose reads are done: LDS keeps the wave's order).
  float* const partial = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * g + i;
    if (r < nr) {
#pragma unroll
      for (int m = 0; m < NT; ++m) partial[(wave * NR + r) * kBlock + 16 * (NT * half + m) + n] = acc[m][i];
    }
  }
  __syncthreads();
  finish_strip<WAVES, WAVES * PARTS>(partial, NR, hw, lane, nr, r0, strip, out_dim, svh, y, y_dtype);
}

template <int BITS, int WAVES, int PARTS>
static hipError_t launch_mfma_bwh(int rows, int in_dim, int out_dim, const uint16_t* z, const uint32_t* trellis,
                                  const uint16_t* svh, void* y, int y_dtype, hipStream_t stream) {
  const dim3 grid(out_dim / kBlock, (rows + kRowsPerPass - 1) / kRowsPerPass);
  hipLaunchKernelGGL((linear_mfma_kernel<BITS, WAVES, PARTS>), grid, dim3(kWave * WAVES * PARTS), 0, stream, z,
                     trellis, svh, y, y_dtype, rows, in_dim, out_dim);
  return hipGetLastError();
}

// The column-split forms run where the first form would put fewer waves than
// the device has SIMDs (1024 on MI355X) in flight, at 4 waves (see
// mfma_column_parts); the choice depends on the shape, never on the rows.
template <int BITS>
static hipError_t launch_mfma_b(int waves, int split, int rows, int in_dim, int out_dim, const uint16_t* z,
                                const uint32_t* trellis, const uint16_t* svh, void* y, int y_dtype,
                                hipStream_t stream) {
  if (waves == 8) return launch_mfma_bwh<BITS, 8, 1>(rows, in_dim, out_dim, z, trellis, svh, y, y_dtype, stream);
  const int parts = split < 0 ? mfma_column_parts(out_dim, waves) : split == 0 ? 1 : 2;
  if (parts == 2) return launch_mfma_bwh<BITS, 4, 2>(rows, in_dim, out_dim, z, trellis, svh, y, y_dtype, stream);
  return launch_mfma_bwh<BITS, 4, 1>(rows, in_dim, out_dim, z, trellis, svh, y, y_dtype, stream);
}

hipError_t launch_linear_mfma(int bits, int waves, int rows, int in_dim, int out_dim, const uint16_t* z,
                              const uint32_t* trellis, const uint16_t* svh, void* y, int y_dtype,
                              hipStream_t stream, int split) {
  if (rows == 0) return hipSuccess;
  switch (bits) {
    case 2: return launch_mfma_b<2>(waves, split, rows, in_dim, out_dim, z, trellis, svh, y, y_dtype, stream);
    case 3: return launch_mfma_b<3>(waves, split, rows, in_dim, out_dim, z, trellis, svh, y, y_dtype, stream);
    case 4: return launch_mfma_b<4>(waves, split, rows, in_dim, out_dim, z, trellis, svh, y, y_dtype, stream);
    case 5: return launch_mfma_b<5>(waves, split, rows, in_dim, out_dim, z, trellis, svh, y, y_dtype, stream);
    case 6: return launch_mfma_b<6>(waves, split, rows, in_dim, out_dim, z, trellis, svh, y, y_dtype, stream);
    default: return launch_mfma_b<8>(waves, split, rows, in_dim, out_dim, z, trellis, svh, y, y_dtype, stream);
  }
}

}  // namespace tf_exl3
