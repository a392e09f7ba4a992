// Device-side helpers shared by the tattn kernels (gfx950 / CDNA4).
//
// Operand layouts of the matrix instructions used here (wave64):
//   v_mfma_f32_32x32x16_bf16: lane l holds A[m = l%32][k = (l/32)*8 + t] and
//     B[k = (l/32)*8 + t][n = l%32], t = 0..7; result register r of lane l is
//     D[m = 8*(r/4) + 4*(l/32) + r%4][n = l%32], r = 0..15.
//   v_mfma_f32_32x32x16_f16 has the same layout with fp16 operands.
//   v_mfma_f32_32x32x64_f8f6f4 (E4M3 x E4M3): lane l holds 32 bytes of row
//     m = l%32 of A and of column n = l%32 of B in the same k positions
//     (group l/32, byte p); the result layout is the one above.
// The kernels compute S^T = K Q^T so that each lane owns one query column and
// softmax statistics stay inside a lane pair (l, l^32).  The contraction over
// keys in P.V pairs the P values a lane already holds with V stored
// transposed and key-permuted to match (see kperm_* below).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace tattn {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLog2_448 = 8.807354922057604f;

// ---------------------------------------------------------------------------
// Key permutation inside a 64-key tile.  In the S^T result of two 32x32
// blocks (keys 32b..32b+31), lane half h holds register r of block b for key
//   key(b, r, h) = 32b + 8(r/4) + 4h + r%4,
// i.e. P value number p = 16b + r of that lane.  The P.V contraction uses the
// lane's own P values as the B operand, so V must be stored with the same key
// order: with K = 16 per instruction (chunk c = p/8), element (2c + h)*8 + p%8
// of a transposed V row.
__host__ __device__ inline int key_p(int key) {  // P index inside its lane half
  return 16 * (key >> 5) + 4 * ((key >> 3) & 3) + (key & 3);
}
__host__ __device__ inline int key_h(int key) { return (key >> 2) & 1; }
__host__ __device__ inline int vt_pos(int key) {
  const int p = key_p(key);
  return (2 * (p >> 3) + key_h(key)) * 8 + (p & 7);
}

// Key blocks of BK <= 8 keys: a step gathers G = 64 / BK blocks (slots), and
//   score row m holds key prow(m) % BK of slot prow(m) / BK,
// where prow(m), m with bits 2 and 3 swapped, is the place of row m's P value
// in the P.V operand order (chunk c = prow / 16, lane half (prow / 8) & 1,
// element prow % 8).  A slot's keys are then BK consecutive P values of one
// lane half, so its maximum needs no exchange between lanes, and with
// BK >= 4 the rows of a slot come in runs of four consecutive score rows,
// which suits the row gathers of K and V.
__host__ __device__ inline int prow(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }
template <int BK>
__host__ __device__ inline int slotg(int m) { return prow(m) / BK; }
template <int BK>
__host__ __device__ inline int kkg(int m) { return prow(m) % BK; }

// Key order of a stored E4M3 V^T row of a 64-key tile (the A operand of the
// fp8 P.V MFMA).  The fp8 MFMA takes 32 bytes per lane in the same k
// positions for A and B; the B operand of a lane (query column, half h) is
// its own 32 probability codes in register order p = 16b + r, i.e. of keys
// 32b + 8(r/4) + 4h + r%4.  Byte 32h + p of V^T row d therefore holds
// V[key][d] of that key.
__host__ __device__ inline int pv8_key(int e) {
  const int h = e >> 5, p = e & 31, r = p & 15;
  return 32 * (p >> 4) + 8 * (r >> 2) + 4 * h + (r & 3);
}

// d permutation of a stored fp8 K row: byte position 64i + 32g + p holds
// d = 64i + 16(p/8) + 8g + p%8, so that a lane (group g) reads its 32 bytes
// for instruction i contiguously, in the order its bf16 Q registers give.
__host__ __device__ inline int k8_pos(int d) {
  const int i = d >> 6, dd = d & 63;
  const int g = (dd >> 3) & 1;
  const int p = 8 * (dd >> 4) + (dd & 7);
  return 64 * i + 32 * g + p;
}

// ---------------------------------------------------------------------------
// E4M3 (OCP) conversion: round to nearest even on the hardware converter.
// The converter does not saturate above 464, so values are clamped first.
template <bool HI>
__device__ inline int cvt_fp8x2(float a, float b, int old) {
  a = __builtin_fminf(__builtin_fmaxf(a, -448.0f), 448.0f);
  b = __builtin_fminf(__builtin_fmaxf(b, -448.0f), 448.0f);
  return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
}

__device__ inline float bf16_to_f32(uint16_t h) { return __uint_as_float(static_cast<uint32_t>(h) << 16); }
__device__ inline uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f)); }
__device__ inline uint16_t f32_to_f16(float f) { return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f)); }

// ---------------------------------------------------------------------------
// MXFP4 (OCP Microscaling): E2M1 elements (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4,
// 6; code = 2 * exponent field + mantissa bit, bit 3 the sign) with one E8M0
// scale 2^e per 32 elements, e = floor(log2 amax) - 2 (2 = the exponent of
// E2M1's largest normal), clamped to [-127, 127]; -127 for an all-zero block.
__device__ inline int mx4_exponent(float amax) {
  if (!(amax > 0.0f)) return -127;
  const int e = ilogbf(amax) - 2;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}
// E2M1 code of y (the element already divided by its block scale, |y| < 8):
// round to nearest, ties to even, on the grid spacing of y's binade (0.5 below
// 2, 1 in [2, 4), 2 above), magnitudes past 6 clamped to 6.  Every candidate
// is computed and one is selected, so the code has no branches (a branchy form
// compiled to divergent regions that spilled registers where it is unrolled).
__device__ inline uint32_t e2m1_code(float y) {
  const float a = __builtin_fabsf(y);
  const float c_lo = __builtin_rintf(a * 2.0f);                        // [0, 2): codes 0..4
  const float c_mid = __builtin_rintf(a) + 2.0f;                       // [2, 4): 2, 3, 4 -> 4, 5, 6
  const float c_hi = __builtin_rintf(a * 0.5f) >= 3.0f ? 7.0f : 6.0f;  // 6 (or 8) -> 7, 4 -> 6
  const float c = a < 2.0f ? c_lo : (a < 4.0f ? c_mid : c_hi);
  return static_cast<uint32_t>(c) | (y < 0.0f ? 8u : 0u);
}

// Value of an E2M1 code (bit 3 the sign): 0, 0.5, 1, 1.5, 2, 3, 4, 6
// (branch-free, as e2m1_code).
__device__ inline float e2m1_value(uint32_t c) {
  const uint32_t m = c & 7u;
  const float sub = 0.5f * static_cast<float>(m);                                     // m = 0, 1
  const float nrm = __builtin_amdgcn_ldexpf(1.0f + 0.5f * static_cast<float>(m & 1u),
                                            static_cast<int>(m >> 1) - 1);            // m >= 2
  const float mag = m < 2u ? sub : nrm;
  return (c & 8u) ? -mag : mag;
}

// ---------------------------------------------------------------------------
// Wave-level reductions (wave64).
__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ inline double wave_max_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ inline double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ inline int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// This lane's index in the wave, read from the hardware where it is used
// (v_mbcnt): address terms formed from it need no register held across a
// kernel, and the volatile asm keeps the compiler from merging the reads.
__device__ inline int lane_here() {
  int l;
  __asm__ volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// Register values made opaque to the optimiser: nothing is hoisted, folded or
// fused across this point.  Each statement holds one real s_nop because the
// compiler's hazard recognizer counts an inline asm statement as one wait
// state: an empty statement placed between an MFMA and a read of its result
// would make it skip nops that the hardware needs.
template <class A>
__device__ inline void opaque(A& a) { __asm__ volatile("s_nop 0" : "+v"(a)); }
template <class A, class B>
__device__ inline void opaque(A& a, B& b) { __asm__ volatile("s_nop 0" : "+v"(a), "+v"(b)); }
template <class A, class B, class C, class E>
__device__ inline void opaque(A& a, B& b, C& c, E& e) {
  __asm__ volatile("s_nop 0" : "+v"(a), "+v"(b), "+v"(c), "+v"(e));
}
template <int N>
__device__ inline void opaque_arr(int (&x)[N]) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8, "opaque_arr: 1, 2, 4 or 8 registers");
  if constexpr (N == 1) opaque(x[0]);
  else if constexpr (N == 2) opaque(x[0], x[1]);
  else if constexpr (N == 4) opaque(x[0], x[1], x[2], x[3]);
  else
    __asm__ volatile("s_nop 0" : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]),
                     "+v"(x[6]), "+v"(x[7]));
}

}  // namespace tattn
