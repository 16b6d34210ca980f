// Device helpers shared by the gfx950 kernels: buffer loads, bf16 unpacking,
// wave64 DPP reductions and MFMA wrappers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace skv {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kBlock = 64;  // tokens per KV block

// Buffer resource over [base, base + bytes).  Loads at or past `bytes` return
// zeros, which is how reads beyond a sequence's end are kept harmless.
// dword3 = 0x00020000: raw 32-bit data format, the gfx9 (CDNA) encoding.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
}

// Streaming (non-temporal) 16-byte load, for data read once in whole
// 128-byte lines: it is not kept in L2, which lets HBM run closer to peak.
// Loads that touch only part of a line per instruction must not use it: the
// rest of the line would be fetched again by the next instruction.
__device__ __forceinline__ u32x4 load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 2 /* nt */);
}

__device__ __forceinline__ float load4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0));
}

// bf16 pair in a dword: element 0 in the low half.
__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// Hardware reciprocal and reciprocal square root (about 1 ulp).
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float fast_rsq(float x) { return __builtin_amdgcn_rsqf(x); }

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}

// All-reduce over each row of 16 lanes; every lane of the row gets the
// result.  The partner pattern (quad swaps, then half-row and row mirrors)
// is symmetric, so all 16 lanes compute bit-identical values.
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp<0xB1>(x));   // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp<0x4E>(x));   // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp<0x141>(x));  // row_half_mirror
  x = fmaxf(x, dpp<0x140>(x));  // row_mirror
  return x;
}

__device__ __forceinline__ float row16_sum(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x141>(x);
  x += dpp<0x140>(x);
  return x;
}

// Sum of x over the lanes that differ only in lane bit 4 (resp. 5): with both
// operands equal, permlane16_swap returns (even rows, odd rows) of 16 lanes
// duplicated in place, permlane32_swap (low half, high half); the two halves'
// sum is identical in every lane.  Pure VALU, no LDS traffic.
__device__ __forceinline__ float xrow16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xhalf_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xrow16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float wave_sum(float x) { return xhalf_sum(xrow16_sum(row16_sum(x))); }
__device__ __forceinline__ float wave_max(float x) { return xhalf_max(xrow16_max(row16_max(x))); }

// Sum over the lanes sharing lane % CPR (the token phases of the row layout):
// lane bits log2(CPR) .. 5.
template <int CPR>
__device__ __forceinline__ float phase_sum(float x) {
  static_assert(CPR == 8 || CPR == 16 || CPR == 32, "chunks per row");
  if constexpr (CPR == 8) x += dpp<0x128>(x);  // row_ror:8 pairs lane l with l ^ 8
  if constexpr (CPR <= 16) x = xrow16_sum(x);
  return xhalf_sum(x);
}

// Orders this wave's LDS writes before its later LDS reads of what other
// lanes of the same wave wrote (and those reads before later overwrites).
// One wave's LDS operations complete in order, so this only stops the
// compiler from moving them; it emits no wait.
__device__ __forceinline__ void wave_lds_exchange() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float readlane(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

// 16x16 output tile of D = A(16 x K) * B(K x 16) + C.  Operand lanes: A row
// and B column = lane % 16, the K slice = lane / 16.  Result: D[i][j] lives
// in lane j + 16 * (i / 4), register i % 4.
__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Geometry of one token row of K or V (d elements of type T) as 16-byte chunks.
template <typename T, int D>
struct Geo {
  static constexpr int ES = sizeof(T);
  static constexpr int ROWB = D * ES;    // bytes per token row
  static constexpr int CPR = ROWB / 16;  // 16-byte chunks per row
  static constexpr int E = 16 / ES;      // elements per chunk
  static constexpr int TPI = 64 / CPR;   // token rows per wave-wide 16-byte load
  static constexpr int NPH = TPI;        // token phases in the row layout
  static constexpr int KA = CPR / 4;     // K chunks per lane per 16-token group
  static_assert(CPR >= 8 && CPR <= 32, "row geometry");
};

template <typename T>
__device__ __forceinline__ float elem_f32(const T* p, int i) {
  if constexpr (sizeof(T) == 2)
    return __uint_as_float((uint32_t)((const uint16_t*)p)[i] << 16);
  else
    return ((const float*)p)[i];
}

// Wave-uniform read of data the kernel never writes (block lists, block
// tables, visit orders) through the scalar cache: it waits on the scalar
// counter only, never on vector loads in flight.  The index must be
// wave-uniform.
__device__ __forceinline__ int32_t uniform_load(const int32_t* p, int64_t i) {
  typedef __attribute__((address_space(4))) const int32_t* const_i32_ptr;
  return ((const_i32_ptr)p)[i];
}

__host__ __device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

}  // namespace skv
