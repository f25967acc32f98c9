// Device helpers shared by the kvsel HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvsel {

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

typedef short short2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ---- bf16 <-> f32 --------------------------------------------------------
// A 32-bit word holding two bf16 values (element 0 in the low half).
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Exact products of two bf16 pairs accumulated in fp32 (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

// ---- transcendental ------------------------------------------------------
// 2^x on the hardware exp unit; callers pre-multiply natural-log arguments by
// log2(e).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }

// ---- cross-lane reductions (DPP within 16-lane rows) ----------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
// DPP controls (gfx9 encoding)
constexpr int kQuadXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;  // lane i <-> 7-i within each half row
constexpr int kRowMirror = 0x140;      // lane i <-> 15-i within each row

// All-reduce (sum) over aligned groups of N lanes, N in {1,2,4,8,16,32,64};
// every lane of the group ends with the group total.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (N >= 2) v += dpp<kQuadXor1>(v);
  if constexpr (N >= 4) v += dpp<kQuadXor2>(v);
  if constexpr (N >= 8) v += dpp<kRowHalfMirror>(v);
  if constexpr (N >= 16) v += dpp<kRowMirror>(v);
  if constexpr (N >= 32) v += __shfl_xor(v, 16, 64);
  if constexpr (N >= 64) v += __shfl_xor(v, 32, 64);
  return v;
}

template <int N>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (N >= 2) v = fmaxf(v, dpp<kQuadXor1>(v));
  if constexpr (N >= 4) v = fmaxf(v, dpp<kQuadXor2>(v));
  if constexpr (N >= 8) v = fmaxf(v, dpp<kRowHalfMirror>(v));
  if constexpr (N >= 16) v = fmaxf(v, dpp<kRowMirror>(v));
  if constexpr (N >= 32) v = fmaxf(v, __shfl_xor(v, 16, 64));
  if constexpr (N >= 64) v = fmaxf(v, __shfl_xor(v, 32, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) { return group_sum<64>(v); }
__device__ __forceinline__ float wave_max(float v) { return group_max<64>(v); }

// 16-byte global loads.  ld16_stream marks the access non-temporal: data
// read exactly once (the K/V stream) should not displace reused lines.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint4 ld16_stream(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
// Non-temporal 16-byte store (results not re-read by this library).
__device__ __forceinline__ void st16_stream(void* p, float4 v) {
  typedef float f32x4v __attribute__((ext_vector_type(4)));
  __builtin_nontemporal_store(f32x4v{v.x, v.y, v.z, v.w}, reinterpret_cast<f32x4v*>(p));
}

// ---- MFMA operands (v_mfma_f32_16x16x32_bf16) ------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Whole-line K fragment loads for v_mfma_f32_16x16x32_bf16.  Its A operand
// gives lane (r = lane & 15, g = lane >> 4) 8 dims of key row r, so the
// fragment of one 32-dim k-step holds 64 bytes of each of 16 rows: every
// load instruction touches 16 half lines.  Two consecutive k-steps 2v and
// 2v + 1 together span bytes [128 v, 128 v + 128) of each row, one line.
// They are loaded as two instructions that each read 8 whole lines: lane
// (r, g) takes 16 bytes at line segment g + 4 (r >> 3) of key r & 7 (first
// load) and of key 8 + (r & 7) (second).  Lane r < 8 then holds its own
// step-2v fragment and lane r + 8's step-2v + 1 fragment; lane r >= 8 the
// reverse.  One DPP row rotation by 8 per dword swaps the misplaced halves.
__device__ __forceinline__ void k_line_exchange(bf16x8& s0, bf16x8& s1, bool lo) {
  uint4 a = __builtin_bit_cast(uint4, s0), c = __builtin_bit_cast(uint4, s1);
  auto ex = [lo](uint32_t& u0, uint32_t& u1) {
    const uint32_t give = lo ? u1 : u0;
    const uint32_t take = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)give, 0x128 /* row_ror:8 */, 0xF, 0xF, false);
    u0 = lo ? u0 : take;
    u1 = lo ? take : u1;
  };
  ex(a.x, c.x);
  ex(a.y, c.y);
  ex(a.z, c.z);
  ex(a.w, c.w);
  s0 = __builtin_bit_cast(bf16x8, a);
  s1 = __builtin_bit_cast(bf16x8, c);
}

}  // namespace kvsel
