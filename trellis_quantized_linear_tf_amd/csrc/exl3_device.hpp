// Device building blocks of the EXL3 decode-row projection for gfx950 (wave64).
//
// The projection is the one the TensorFold pull request "hip exl3: the input
// rotation and trellis linear for decode rows" describes in "What this
// changes"; the stream format and rounding rules are stated in tf_exl3.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tf_exl3 {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kBlock = 128;               // rotation block and output strip width
constexpr int kRowsPerPass = 16;
constexpr uint32_t kHashMul = 0x9E3779u;  // < 2^24, so v_mul_u32_u24 is exact
constexpr uint32_t kScaleBits = 0x3DB504F3u;  // RN32(1/sqrt(128))
constexpr uint32_t kCbScale = 0x1EEEu;    // fp16 A
constexpr uint32_t kCbBias = 0xC931u;     // fp16 B

__device__ __forceinline__ float bits_to_f32(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t f32_to_bits(float f) { return __builtin_bit_cast(uint32_t, f); }

// Keeps the compiler from fusing an fp32 value into its consumer (a multiply
// followed by an fp16 convert would otherwise become one v_fma_mix rounding).
__device__ __forceinline__ float opaque(float v) {
  asm volatile("" : "+v"(v));
  return v;
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float v) {
  const _Float16 h = (_Float16)v;  // v_cvt_f16_f32, round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) { return bits_to_f32((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest even; a NaN stays a quiet NaN of the same sign.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float v) {
  uint32_t u = f32_to_bits(v);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---------------------------------------------------------------------------
// Codebook: two 16-bit states -> two packed fp16 weights.
//   x = state * 0x9E3779 (low 32 bits); h = byte sum of x;
//   w = fma(1024 + h, A, B) in fp16, one rounding.
// 1024 + h is the fp16 whose bits are 0x6400 + h (h <= 1020 keeps it in
// [1024, 2048)), so the byte sums land directly in packed fp16 form: v_sad_u8
// adds the first sum to 0x64006400 and v_sad_hi_u8 adds the second sum shifted
// into the top half; one v_pk_fma_f16 then finishes both values.
__device__ __forceinline__ half2_t decode_pair(uint32_t s0, uint32_t s1) {
  const uint32_t x0 = __umul24(s0, kHashMul);
  const uint32_t x1 = __umul24(s1, kHashMul);
  uint32_t t = __builtin_amdgcn_sad_u8(x0, 0u, 0x64006400u);
  t = __builtin_amdgcn_sad_hi_u8(x1, 0u, t);
  const half2_t v = __builtin_bit_cast(half2_t, t);
  const half2_t a = __builtin_bit_cast(half2_t, kCbScale * 0x10001u);
  const half2_t b = __builtin_bit_cast(half2_t, kCbBias * 0x10001u);
  return __builtin_elementwise_fma(v, a, b);
}

// 16-bit window starting at bit i*BITS of the little-endian word array w[]
// (i is a constant after unrolling, so the word index and shift fold away).
template <int BITS>
__device__ __forceinline__ uint32_t window_at(const uint32_t* w, int i) {
  const int o = i * BITS;
  const int d = o >> 5;
  const int sh = o & 31;
  const uint32_t v = (sh <= 16) ? (w[d] >> sh) : __builtin_amdgcn_alignbit(w[d + 1], w[d], sh);
  return v & 0xFFFFu;
}

// Funnel shift: bits [sh, sh + 32) of the 64-bit value hi:lo. Kept opaque so
// the compiler does not narrow it when only one half of the result is used.
template <int SH>
__device__ __forceinline__ uint32_t funnel(uint32_t hi, uint32_t lo) {
  uint32_t r;
  asm("v_alignbit_b32 %0, %1, %2, %3" : "=v"(r) : "v"(hi), "v"(lo), "i"(SH));
  return r;
}

// The 32 states of a lane's share (see decode_lane); w[BITS] is the next
// lane's first dword. When BITS divides 16 the
// window at offset o + 16 is the top half of the funnel shift that gives the
// window at o, so one shift serves two states; the 16-bit halves then reach
// v_mul_u32_u24 through its WORD_0 / WORD_1 operand selects at no cost.
template <int BITS, int I = 0>
__device__ __forceinline__ void lane_states(const uint32_t (&w)[BITS + 1], uint32_t (&st)[32]) {
  if constexpr (I < 32) {
    constexpr int o = I * BITS;
    constexpr int d = o >> 5;
    constexpr int sh = o & 31;
    if constexpr (16 % BITS == 0) {
      if constexpr (sh < 16) {
        uint32_t t;
        if constexpr (sh == 0) {
          t = w[d];
        } else {
          t = funnel<sh>(w[d + 1], w[d]);
        }
        st[I] = t & 0xFFFFu;
        st[I + 16 / BITS] = t >> 16;
      }
    } else {
      st[I] = window_at<BITS>(w, I);
    }
    lane_states<BITS, I + 1>(w, st);
  }
}

// Lane that holds the dword following this lane's share inside the same tile.
__device__ __forceinline__ int next_lane_in_tile(int lane) { return (lane & ~7) | ((lane + 1) & 7); }

// `v` of lane next_lane_in_tile(this lane), through the LDS crossbar (no LDS
// memory is touched).
__device__ __forceinline__ uint32_t next_lane_word(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_ds_bpermute(next_lane_in_tile(__lane_id()) * 4, (int)v);
}

// A lane's share of one tile row of a 128-column strip. The strip's tile row is
// 8 tiles of 32*BITS bytes, contiguous; lane = 8t + q holds the BITS dwords at
// bits 32*BITS*q .. of tile t, which are tile values 32q .. 32q+31 = strip
// columns 2*lane and 2*lane+1, 16 k values each. The last windows reach at most
// 16 - BITS bits past the lane's own bits, into the next lane's first dword
// (within the tile, q = 7 wrapping to q = 0), which comes across with one
// ds_bpermute: a second load of it would double the wave's memory instructions.
// Every lane of the wave must be active.
// Output: wp[c][p] = packed (W[2p][2*lane+c], W[2p+1][2*lane+c]) of the tile row.
template <int BITS>
__device__ __forceinline__ void decode_lane(const uint32_t (&w)[BITS], half2_t (&wp)[2][8]) {
  uint32_t we[BITS + 1];
#pragma unroll
  for (int i = 0; i < BITS; ++i) we[i] = w[i];
  we[BITS] = next_lane_word(w[0]);
  uint32_t st[32];
  lane_states<BITS>(we, st);
#pragma unroll
  for (int c = 0; c < 2; ++c) {
#pragma unroll
    for (int p = 0; p < 8; ++p) wp[c][p] = decode_pair(st[16 * c + 2 * p], st[16 * c + 2 * p + 1]);
  }
}

// One column of a tile: its 16 values' states. u[] holds the column's bits
// starting at bit 0 (value 0's window) and the 16 - BITS bits after them; the
// windows sit at bits j*BITS, j = 0..15 (the same funnel-pair rule as
// lane_states when BITS divides 16).
template <int BITS>
constexpr int column_words() {
  return (16 * BITS + 16 - BITS + 31) / 32;
}

template <int BITS, int I = 0>
__device__ __forceinline__ void column_states(const uint32_t (&u)[column_words<BITS>()], uint32_t (&st)[16]) {
  if constexpr (I < 16) {
    constexpr int o = I * BITS;
    constexpr int d = o >> 5;
    constexpr int sh = o & 31;
    if constexpr (16 % BITS == 0) {
      if constexpr (sh < 16) {
        uint32_t t;
        if constexpr (sh == 0) {
          t = u[d];
        } else {
          t = funnel<sh>(u[d + 1], u[d]);
        }
        st[I] = t & 0xFFFFu;
        if constexpr (I + 16 / BITS < 16) st[I + 16 / BITS] = t >> 16;
      }
    } else {
      st[I] = window_at<BITS>(u, I);
    }
    column_states<BITS, I + 1>(u, st);
  }
}

// The column's weights as packed (k, k+1) pairs: wp[p] = (W[2p][col], W[2p+1][col]).
template <int BITS>
__device__ __forceinline__ void decode_column(const uint32_t (&u)[column_words<BITS>()], half2_t (&wp)[8]) {
  uint32_t st[16];
  column_states<BITS>(u, st);
#pragma unroll
  for (int p = 0; p < 8; ++p) wp[p] = decode_pair(st[2 * p], st[2 * p + 1]);
}

// ---------------------------------------------------------------------------
// The value lane ^ H holds, for the butterfly stages. DPP moves inside the
// VALU where gfx950 has the pattern (H = 1, 2: quad_perm; H = 8: row_ror:8,
// which is lane ^ 8 inside each 16-lane row), ds_swizzle's xor mode (no
// address register) for H = 4 and 16, and a bpermute across the two 32-lane
// halves for H = 32. Every lane of the wave must be active.
template <int H>
__device__ __forceinline__ float lane_xor(float v) {
  const int i = __builtin_bit_cast(int, v);
  int r;
  if constexpr (H == 1) {
    r = __builtin_amdgcn_mov_dpp(i, 0xB1, 0xF, 0xF, false);  // quad_perm [1, 0, 3, 2]
  } else if constexpr (H == 2) {
    r = __builtin_amdgcn_mov_dpp(i, 0x4E, 0xF, 0xF, false);  // quad_perm [2, 3, 0, 1]
  } else if constexpr (H == 8) {
    r = __builtin_amdgcn_mov_dpp(i, 0x128, 0xF, 0xF, false);  // row_ror:8
  } else if constexpr (H == 4 || H == 16) {
    r = __builtin_amdgcn_ds_swizzle(i, 0x1F | (H << 10));  // and 0x1F, or 0, xor H
  } else {
    r = __builtin_bit_cast(int, __shfl_xor(v, H));
  }
  return __builtin_bit_cast(float, r);
}

// One stage h < 64: the pair (i, i + h) becomes (a + b, a - b) rounded to fp32;
// a lane in the upper half of a pair computes fma(v, -1, partner) = partner - v
// exactly as a subtraction would (v * -1 is exact, one rounding follows).
template <int H>
__device__ __forceinline__ void fwht_stage(float& v0, float& v1, int lane) {
  const float sgn = (lane & H) ? -1.0f : 1.0f;
  const float p0 = lane_xor<H>(v0);
  const float p1 = lane_xor<H>(v1);
  v0 = __builtin_fmaf(v0, sgn, p0);
  v1 = __builtin_fmaf(v1, sgn, p1);
}

// 128-point butterflies on one wave: element e of the block lives in lane e % 64,
// register e / 64 (v0 holds e = lane, v1 holds e = lane + 64). Stages run
// h = 1, 2, ..., 64; stages 1..32 pair lanes lane ^ h (fwht_stage); stage 64
// pairs v0 with v1 inside the lane.
__device__ __forceinline__ void fwht128_wave(float& v0, float& v1) {
  const int lane = __lane_id();
  fwht_stage<1>(v0, v1, lane);
  fwht_stage<2>(v0, v1, lane);
  fwht_stage<4>(v0, v1, lane);
  fwht_stage<8>(v0, v1, lane);
  fwht_stage<16>(v0, v1, lane);
  fwht_stage<32>(v0, v1, lane);
  const float a = v0;
  const float b = v1;
  v0 = a + b;
  v1 = a - b;
}

// ---------------------------------------------------------------------------
// rot_in on one 128-block held by one wave: lane l gets elements l and l + 64.
//   p = RN32(x * suh); butterflies (fwht128_wave); RN32(p * s); RN16 once.
// The fp32 values pass an empty register barrier after the product and after
// the scale, so neither is fused into its consumer (no single-rounding
// multiply-and-convert). Both the rot_in kernel and the fused projection call
// this, so they produce the same bits.
template <int XDT>
__device__ __forceinline__ float load_in(const void* __restrict__ x, size_t i) {
  if constexpr (XDT == 0) {  // TF_DT_F32
    return static_cast<const float*>(x)[i];
  } else if constexpr (XDT == 1) {  // TF_DT_F16
    return f16_bits_to_f32(static_cast<const uint16_t*>(x)[i]);
  } else {  // TF_DT_BF16
    return bf16_bits_to_f32(static_cast<const uint16_t*>(x)[i]);
  }
}

// The arithmetic after the loads: p = RN32(x * suh), butterflies, RN32(p * s), RN16.
__device__ __forceinline__ void rot_in_math(float x0, float x1, float g0, float g1, uint16_t& z0, uint16_t& z1) {
  float v0 = opaque(x0 * g0);
  float v1 = opaque(x1 * g1);
  fwht128_wave(v0, v1);
  const float s = bits_to_f32(kScaleBits);
  v0 = opaque(v0 * s);
  v1 = opaque(v1 * s);
  z0 = f32_to_f16_bits(v0);
  z1 = f32_to_f16_bits(v1);
}

// x + base is the block's first element, suh + col0 its first sign.
template <int XDT>
__device__ __forceinline__ void rot_in_block(const void* __restrict__ x, size_t base,
                                             const uint16_t* __restrict__ suh, int col0, int lane,
                                             uint16_t& z0, uint16_t& z1) {
  rot_in_math(load_in<XDT>(x, base + lane), load_in<XDT>(x, base + lane + 64),
              f16_bits_to_f32(suh[col0 + lane]), f16_bits_to_f32(suh[col0 + lane + 64]), z0, z1);
}

// Raw element of x (fp32 bits, or fp16/bf16 bits) and its widening, split so a
// wave can issue the loads of several blocks before using any of them.
__device__ __forceinline__ uint32_t load_raw(const void* __restrict__ x, int x_dtype, size_t i) {
  return x_dtype == 0 ? static_cast<const uint32_t*>(x)[i] : (uint32_t) static_cast<const uint16_t*>(x)[i];
}

__device__ __forceinline__ float widen_raw(uint32_t v, int x_dtype) {
  return x_dtype == 0 ? bits_to_f32(v) : x_dtype == 1 ? f16_bits_to_f32((uint16_t)v) : bf16_bits_to_f32((uint16_t)v);
}

}  // namespace tf_exl3
