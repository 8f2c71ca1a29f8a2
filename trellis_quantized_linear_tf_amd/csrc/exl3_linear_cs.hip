// Column-split variant of the v_dot2 linear, for narrow matrices.
//
// TensorFold pull request "hip exl3: the input rotation and trellis linear for
// decode rows", "What this changes": the sums are v_dot2_f32_f16 chains in a
// fixed order set by the wave count. A matrix with few 128-column strips (the
// page's Engram layers have 200, the indexer one) gives the regular kernel too
// few waves to fill 1024 SIMDs, and one wave per SIMD cannot hide its own
// instruction latencies. Here each strip's workgroup has twice the waves: half
// h = 0, 1 takes strip columns 64h .. 64h+63, one column per lane, and within
// a half the waves split the tile rows exactly as the regular kernel's WAVES
// waves do. A lane decodes its column's 16 values per tile row and runs that
// column's chain: the same decoded pairs, the same z pairs, the same
// v_dot2_f32_f16 sequence and the same cross-wave sum order as the regular
// kernel's lane that owns the column, so the outputs are bit-identical.
//
// Lane l of half h owns column n = l % 16 of tile t = 4h + l / 16. A column's 16
// values are tile bits [16 * n * bits, 16 * (n + 1) * bits), and its last
// windows reach 16 - bits bits further (into the next column, wrapping inside
// the tile). The lane loads the dwords covering that span (nontemporal, wave
// loads coalesce to the tile); at odd widths an odd column starts 16 bits into
// its first dword, and one funnel shift per dword realigns it. The row inputs
// of a step go through a wave-private LDS slot (as in linear_lds_kernel).
#include "exl3_launch.hpp"
#include "exl3_strip.hpp"

namespace tf_exl3 {

template <int BITS, int WAVES, int NR>
__global__ __launch_bounds__(kWave * 2 * WAVES) void linear_cs_kernel(const uint16_t* __restrict__ z,
                                                                      const uint32_t* __restrict__ trellis,
                                                                      const uint16_t* __restrict__ svh,
                                                                      void* __restrict__ y, int y_dtype, int rows,
                                                                      int in_dim, int out_dim, int layout) {
  // Twice the regular kernel's tile rows in flight: a narrow launch has about two
  // waves per SIMD, so each wave must carry twice the stream bytes in flight for the
  // device to hold as many as the latency of HBM asks for (vector registers are
  // plentiful at this occupancy). Passes of 2 and 4 rows keep the regular depth:
  // their scalar z loads for the longer unrolled ring would not fit the SGPRs.
  constexpr int PF = (NR == 1 || NR > kScalarZRows ? 2 : 1) * prefetch_depth<BITS>();
  constexpr int RING = PF + 1;
  constexpr int CW = column_words<BITS>();
  constexpr int ND = BITS % 2 ? CW + 1 : CW;  // dwords loaded per lane
  constexpr int TW = 8 * BITS;                // words per tile
  constexpr int FR = NR < kRowsPerPass ? NR : kRowsPerPass;
  __shared__ float partial[WAVES * FR * kBlock];
  __shared__ uint4 zslot[2 * WAVES][2 * NR];  // per wave: row r, k-half h at [2r + h]

  const int lane = __lane_id();
  const int hw = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = hw >= WAVES ? 1 : 0;
  const int wave = hw - half * WAVES;  // the tile-row split, as in the regular kernel
  const int strip = blockIdx.x;
  const int r0 = blockIdx.y * NR;
  const int nr = min(NR, rows - r0);
  const int iters = in_dim / 16 / WAVES;

  const StreamStrides st = stream_strides<BITS>(layout, in_dim, out_dim);
  const uint32_t* __restrict__ tp = trellis + (size_t)wave * st.row + (size_t)strip * st.strip;
  const size_t step_words = (size_t)WAVES * st.row;
  auto share = [&](int i) { return tp + (size_t)min(i, iters - 1) * step_words; };

  const int t = 4 * half + (lane >> 4);
  const int n = lane & 15;
  const int d0 = (n * BITS) >> 1;                   // the column's first dword in its tile
  const uint32_t shl = (n * BITS) & 1 ? 16u : 0u;   // its first bit in that dword
  int offw[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) offw[i] = t * TW + (d0 + i) % TW;

  const bool stager = lane < 2 * NR;
  const uint4* __restrict__ zsrc = reinterpret_cast<const uint4*>(
      z + (size_t)(r0 + min(lane >> 1, nr - 1)) * in_dim + wave * 16 + (lane & 1) * 8);
  auto zload = [&](int i) { return zsrc[(size_t)min(i, iters - 1) * (WAVES * 2)]; };
  uint4* slot = zslot[hw];

  float acc[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) acc[r] = 0.0f;

  uint32_t ring[RING][ND];
  auto load = [&](uint32_t(&dst)[ND], const uint32_t* p) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < ND; ++i) dst[i] = __builtin_nontemporal_load(p + offw[i]);
  };
  // The column's 16 weights of ring slot D as (k, k+1) pairs.
  auto decode = [&](const uint32_t(&w)[ND], half2_t(&wp)[8]) __attribute__((always_inline)) {
    uint32_t u[CW];
#pragma unroll
    for (int j = 0; j < CW; ++j) {
      if constexpr (BITS % 2) {
        u[j] = __builtin_amdgcn_alignbit(w[j + 1], w[j], shl);
      } else {
        u[j] = w[j];
      }
    }
    decode_column<BITS>(u, wp);
  };

  if constexpr (NR <= kScalarZRows) {
    // Up to 4 rows: the step's z pairs are wave-uniform scalar loads, the SGPR
    // operand of v_dot2c (as in linear_kernel); no LDS slot, no branch, so one
    // step's chain can overlap the next step's decode.
    const uint32_t* zrow[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r)
      zrow[r] = reinterpret_cast<const uint32_t*>(z + (size_t)(r0 + min(r, nr - 1)) * in_dim) + wave * 8;
#pragma unroll
    for (int d = 0; d < PF; ++d) load(ring[d], share(d));
    auto step = [&](auto dc, int i) __attribute__((always_inline)) {
      constexpr int D = decltype(dc)::value;
      load(ring[(D + PF) % RING], share(i + PF));
      half2_t wp[8];
      decode(ring[D], wp);
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const uint32_t* zp = zrow[r] + (size_t)i * (WAVES * 8);
#pragma unroll
        for (int p = 0; p < 8; ++p)
          acc[r] = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, zp[p]), wp[p], acc[r], false);
      }
    };
    step_loop<RING>(iters, step);
  } else {
    uint4 zn = zload(0);
#pragma unroll
    for (int d = 0; d < PF; ++d) load(ring[d], share(d));

    auto step = [&](auto dc, int i) __attribute__((always_inline)) {
      constexpr int D = decltype(dc)::value;
      const uint4 zc = zn;
      zn = zload(i + 1);  // issued before the next stream load: loads complete in order
      load(ring[(D + PF) % RING], share(i + PF));
      if (stager) slot[lane] = zc;
      half2_t wp[8];
      decode(ring[D], wp);
      // Row r + 1's z is read while row r's chain runs (see linear_lds_kernel).
      uint4 lo = slot[0];
      uint4 hi = slot[1];
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const uint32_t zp[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        if (r + 1 < NR) {
          lo = slot[2 * r + 2];
          hi = slot[2 * r + 3];
        }
#pragma unroll
        for (int p = 0; p < 8; ++p)
          acc[r] = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, zp[p]), wp[p], acc[r], false);
        asm volatile("" : "+v"(acc[r])::"memory");
      }
    };
    step_loop<RING>(iters, step);
  }

  // Wave (h, w)'s sums go to partial[w][row][64h + lane]; the finish adds the
  // WAVES tile-row waves in order, FR rows per round.
  const int col = 64 * half + lane;
#pragma unroll
  for (int c = 0; c < NR; c += FR) {
    if (c >= nr) break;  // block-uniform
    if (c > 0) __syncthreads();  // the previous round has read partial
#pragma unroll
    for (int r = 0; r < FR; ++r) partial[(wave * FR + r) * kBlock + col] = acc[c + r];
    __syncthreads();
    finish_strip<WAVES, 2 * WAVES>(partial, FR, hw, lane, min(FR, nr - c), r0 + c, strip, out_dim, svh, y,
                                   y_dtype);
  }
}

template <int BITS, int WAVES, int NR>
static void launch_cs_nr(dim3 grid, const uint16_t* z, const uint32_t* trellis, const uint16_t* svh, void* y,
                         int y_dtype, int rows, int in_dim, int out_dim, int layout, hipStream_t stream) {
  hipLaunchKernelGGL((linear_cs_kernel<BITS, WAVES, NR>), grid, dim3(kWave * 2 * WAVES), 0, stream, z, trellis,
                     svh, y, y_dtype, rows, in_dim, out_dim, layout);
}

template <int BITS, int WAVES>
static void launch_cs_w(int nr_cap, dim3 grid, const uint16_t* z, const uint32_t* trellis, const uint16_t* svh,
                        void* y, int y_dtype, int rows, int in_dim, int out_dim, int layout, hipStream_t stream) {
  switch (nr_cap) {
    case 1: launch_cs_nr<BITS, WAVES, 1>(grid, z, trellis, svh, y, y_dtype, rows, in_dim, out_dim, layout, stream); break;
    case 2: launch_cs_nr<BITS, WAVES, 2>(grid, z, trellis, svh, y, y_dtype, rows, in_dim, out_dim, layout, stream); break;
    case 4: launch_cs_nr<BITS, WAVES, 4>(grid, z, trellis, svh, y, y_dtype, rows, in_dim, out_dim, layout, stream); break;
    case 8: launch_cs_nr<BITS, WAVES, 8>(grid, z, trellis, svh, y, y_dtype, rows, in_dim, out_dim, layout, stream); break;
    case 12: launch_cs_nr<BITS, WAVES, 12>(grid, z, trellis, svh, y, y_dtype, rows, in_dim, out_dim, layout, stream); break;
    default: launch_cs_nr<BITS, WAVES, 16>(grid, z, trellis, svh, y, y_dtype, rows, in_dim, out_dim, layout, stream); break;
  }
}

template <int BITS>
static void launch_cs_b(int waves, int nr_cap, dim3 grid, const uint16_t* z, const uint32_t* trellis,
                        const uint16_t* svh, void* y, int y_dtype, int rows, int in_dim, int out_dim, int layout,
                        hipStream_t stream) {
  if (waves == 8) {
    launch_cs_w<BITS, 8>(nr_cap, grid, z, trellis, svh, y, y_dtype, rows, in_dim, out_dim, layout, stream);
  } else {
    launch_cs_w<BITS, 4>(nr_cap, grid, z, trellis, svh, y, y_dtype, rows, in_dim, out_dim, layout, stream);
  }
}

void launch_linear_cs(int bits, int waves, int nr_cap, dim3 grid, const uint16_t* z, const uint32_t* trellis,
                      const uint16_t* svh, void* y, int y_dtype, int rows, int in_dim, int out_dim, int layout,
                      hipStream_t stream) {
  switch (bits) {
    case 2: launch_cs_b<2>(waves, nr_cap, grid, z, trellis, svh, y, y_dtype, rows, in_dim, out_dim, layout, stream); break;
    case 3: launch_cs_b<3>(waves, nr_cap, grid, z, trellis, svh, y, y_dtype, rows, in_dim, out_dim, layout, stream); break;
    case 4: launch_cs_b<4>(waves, nr_cap, grid, z, trellis, svh, y, y_dtype, rows, in_dim, out_dim, layout, stream); break;
    case 5: launch_cs_b<5>(waves, nr_cap, grid, z, trellis, svh, y, y_dtype, rows, in_dim, out_dim, layout, stream); break;
    case 6: launch_cs_b<6>(waves, nr_cap, grid, z, trellis, svh, y, y_dtype, rows, in_dim, out_dim, layout, stream); break;
    default: launch_cs_b<8>(waves, nr_cap, grid, z, trellis, svh, y, y_dtype, rows, in_dim, out_dim, layout, stream); break;
  }
}

}  // namespace tf_exl3
