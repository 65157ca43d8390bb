// Device-side helpers shared by the attention-state-memory kernels (gfx950,
// wave64).  Nothing here is method-specific arithmetic beyond the packed
// argmax key and the bf16 unpacking.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <math.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define ASM_LOG2E 1.4426950408889634f
#define ASM_LN2 0.6931471805599453f

namespace asmk {

constexpr int kWave = 64;

// ---- bf16 / f32 element access -------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <typename T>
__device__ __forceinline__ float load_elem(const T* p, size_t i);
template <>
__device__ __forceinline__ float load_elem<float>(const float* p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const uint16_t* p, size_t i) {
  return __uint_as_float(uint32_t(p[i]) << 16);
}

// 8 consecutive bf16 (16 bytes, 16-byte aligned) as an MFMA operand.
__device__ __forceinline__ u32x4 ld16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Raw buffer resources: loads address base + voffset + soffset, and any
// 16-byte load at or past num_records bytes returns zeros instead of touching
// memory.  Ragged tails therefore need neither clamping nor branches, and the
// per-lane offsets stay 32-bit and loop-invariant.
constexpr int kBufferFlags = 0x00020000;  // raw buffer, 32-bit data format
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t num_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, int(num_bytes), kBufferFlags);
}
// Marks a wave-uniform pointer as such, so that buffer resources built from
// it live in scalar registers (otherwise every load through them becomes a
// per-lane waterfall loop).
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(u));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(u >> 32));
  return reinterpret_cast<T*>((uint64_t(hi) << 32) | lo);
}
__device__ __forceinline__ u32x4 buf16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}
__device__ __forceinline__ float buf_f32(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}
// The same loads with the non-temporal hint (cache-policy bit nt): for data
// read once per call (the centroid table, the local K/V), which should not
// displace reused lines.  A plain read stream of a few hundred MB runs about
// 12% faster this way on gfx950.
constexpr int kNonTemporal = 2;
__device__ __forceinline__ u32x4 buf16_nt(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kNonTemporal);
}
__device__ __forceinline__ float buf_f32_nt(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, kNonTemporal));
}

// Round a float64 to bf16, nearest with ties to even, in one step (no
// intermediate float32 rounding).  bf16 keeps 8 significant bits and the
// float32 exponent range; values whose rounded magnitude reaches 2^128
// become infinity.
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double x) {
  if (isnan(x)) return 0x7FC0;
  const uint64_t u = __double_as_longlong(x);
  const uint16_t sign = uint16_t((u >> 48) & 0x8000u);
  const double ax = fabs(x);
  if (ax == 0.0) return sign;
  int e;
  frexp(ax, &e);                        // ax = m * 2^e, 0.5 <= m < 1
  int qe = e - 8;                       // spacing of bf16 values near ax
  if (qe < -133) qe = -133;             // subnormal spacing floor
  const double q = ldexp(1.0, qe);
  const double r = rint(ax / q) * q;    // exact division; rint: ties to even
  if (r >= 0x1p128) return sign | 0x7F80;
  const uint32_t b32 = __float_as_uint(float(r));  // exact: r has <= 8 significant bits
  return sign | uint16_t(b32 >> 16);
}

// ---- argmax keys -----------------------------------------------------------
// A score s and index k pack into one 64-bit key whose unsigned order is
// (s ascending, k descending): the maximum key is the highest score, lowest
// index among exact ties.  -0 is folded into +0 first.

__device__ __forceinline__ uint32_t ordered_bits(float s) {
  s = s + 0.0f;
  const uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ uint64_t argmax_key(float s, uint32_t k) {
  return (uint64_t(ordered_bits(s)) << 32) | uint64_t(0xFFFFFFFFu - k);
}
__device__ __forceinline__ uint32_t key_index(uint64_t key) {
  return 0xFFFFFFFFu - uint32_t(key & 0xFFFFFFFFull);
}
__device__ __forceinline__ float key_score(uint64_t key) {
  const uint32_t o = uint32_t(key >> 32);
  const uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __uint_as_float(u);
}
__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// ---- wave shuffles -------------------------------------------------------

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, kWave); }
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  const uint32_t lo = __shfl_xor(uint32_t(v), m, kWave);
  const uint32_t hi = __shfl_xor(uint32_t(v >> 32), m, kWave);
  return (uint64_t(hi) << 32) | lo;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = umax64(v, shfl_xor_u64(v, m));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += shfl_xor_f(v, m);
  return v;
}
__device__ __forceinline__ float readlane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Reductions across the 16 lanes of a DPP row (lanes 16r .. 16r+15) with DPP
// moves instead of LDS permutes: quad swaps, then rotations by 4 and 8.  Every
// lane of the row ends with the row's maximum; for the sum only the value
// read back from one lane is used.
template <int kCtrl>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}
constexpr int kDppQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppRowRor8 = 0x128;
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_mov<kDppQuadXor1>(v));
  v = fmaxf(v, dpp_mov<kDppQuadXor2>(v));
  v = fmaxf(v, dpp_mov<kDppRowRor4>(v));
  v = fmaxf(v, dpp_mov<kDppRowRor8>(v));
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_mov<kDppQuadXor1>(v);
  v += dpp_mov<kDppQuadXor2>(v);
  v += dpp_mov<kDppRowRor4>(v);
  v += dpp_mov<kDppRowRor8>(v);
  return v;
}

// Maximum and sum over the four 16-lane groups of a wave (lanes j, j+16,
// j+32, j+48), with the two lane-swap instructions of gfx950 instead of LDS
// permutes.
__device__ __forceinline__ float group4_max(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const float y = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  const unsigned v = __float_as_uint(y);
  const auto t = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
}
__device__ __forceinline__ float group4_sum(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const float y = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  const unsigned v = __float_as_uint(y);
  const auto t = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}

// Transposing LDS read (gfx950 ds_read_b64_tr_b16) of a row-major tile of
// 16-bit values with `pitch` bytes per row: the matrix-core operand holding,
// in lane (r16, grp), column 16*dt + r16 of rows kb .. kb+3 followed by rows
// kb2 .. kb2+3 (kb, kb2 chosen per lane group).  Over one 16-lane group, lane
// i addresses row kb + i / 4, columns 16*dt + 4*(i % 4) .. +3, and lane j
// receives column 16*dt + j of the four rows.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
__device__ __forceinline__ u32x4 lds_read_colT(const char* base, int pitch, int dt, int kb, int kb2,
                                               int r16) {
  const int roff = (r16 >> 2) * pitch + (16 * dt + 4 * (r16 & 3)) * 2;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + kb * pitch + roff));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + kb2 * pitch + roff));
  return u32x4{__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
               __builtin_bit_cast(u32x2, hi)[0], __builtin_bit_cast(u32x2, hi)[1]};
}

// Orders LDS traffic between lanes of one wave without a workgroup barrier.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__host__ __device__ constexpr size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace asmk
