// Device helpers shared by the gfx950 kernels: element types, conversions,
// 16-byte vector moves and wavefront (64-lane) reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <type_traits>
#include <utility>
#include <stdint.h>

namespace pa {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Storage element tags.  bf16 values are carried as raw 16-bit patterns.
struct F32 { typedef float storage; static constexpr int bytes = 4; };
struct F16 { typedef _Float16 storage; static constexpr int bytes = 2; };
struct BF16 { typedef uint16_t storage; static constexpr int bytes = 2; };

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// fp32 -> bf16, round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}
typedef float f32x2 __attribute__((ext_vector_type(2)));
// Two fp32 values -> packed pair, round to nearest even, one instruction
// (v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), bf16x2));
}
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), f16x2));
}

__device__ __forceinline__ u32x4 ld16(const void *p) {
  return *reinterpret_cast<const u32x4 *>(p);
}
__device__ __forceinline__ void st16(void *p, u32x4 v) { *reinterpret_cast<u32x4 *>(p) = v; }
// Non-temporal 16-byte load (nt cache policy): for data streamed once, such
// as K/V pages in decode.  On MI355X a read stream of such loads sustains
// about 10% more HBM bandwidth than the same stream of plain loads.
__device__ __forceinline__ u32x4 ld16_nt(const void *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

// ---- DPP lane exchange inside a row of 16 lanes ---------------------------
// quad_perm [1,0,3,2] and [2,3,0,1], row_half_mirror, row_mirror.  Each step
// combines a lane with one partner; after the four steps every lane of the
// row holds the same total (each pairwise sum has the same two operands, so
// the lanes agree bit for bit).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
      0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
constexpr int kDppXor1 = 0xB1;
constexpr int kDppXor2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

// Value of the lane 8 apart inside a row (row_ror:8: lane i reads lane
// (i + 8) mod 16 of its row, which is i ^ 8).
constexpr int kDppRor8 = 0x128;

// The values of lanes l and l ^ 16 (l ^ 32) as a pair, by one VALU permute
// (v_permlane16_swap / v_permlane32_swap of two copies of the value).  Both
// lanes of a pair receive the two values in the same order, so a sum of the
// pair is bit-identical on both.  (The two results are copied to scalars
// before the bit cast: a bit cast of an indexed vector element miscompiles,
// every index reading element 0.)
__device__ __forceinline__ f32x2 pair_xor16(float v) {
  const uint32_t a = __builtin_bit_cast(uint32_t, v);
  const auto r = __builtin_amdgcn_permlane16_swap(a, a, false, false);
  const uint32_t r0 = r[0], r1 = r[1];
  return f32x2{__uint_as_float(r0), __uint_as_float(r1)};
}
__device__ __forceinline__ f32x2 pair_xor32(float v) {
  const uint32_t a = __builtin_bit_cast(uint32_t, v);
  const auto r = __builtin_amdgcn_permlane32_swap(a, a, false, false);
  const uint32_t r0 = r[0], r1 = r[1];
  return f32x2{__uint_as_float(r0), __uint_as_float(r1)};
}

__device__ __forceinline__ float shfl_xor(float v, int mask) {
  const int lane = __lane_id();
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(
      (lane ^ mask) << 2, __builtin_bit_cast(int, v)));
}

// Sum over aligned groups of N lanes (N = 8, 16, 32, 64); every lane of a
// group receives the group total.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(N == 8 || N == 16 || N == 32 || N == 64, "group size");
  v += dpp<kDppXor1>(v);
  v += dpp<kDppXor2>(v);
  v += dpp<kDppHalfMirror>(v);
  if constexpr (N >= 16) v += dpp<kDppMirror>(v);
  if constexpr (N >= 32) { const f32x2 r = pair_xor16(v); v = r[0] + r[1]; }
  if constexpr (N >= 64) { const f32x2 r = pair_xor32(v); v = r[0] + r[1]; }
  return v;
}

// NaN-propagating maximum (IEEE maximum): lowers to v_maximum*_f32 without
// the operand canonicalisation an IEEE fmax needs.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Max over lanes that differ only in the bits of STRIDE..32 (i.e. combine
// the 64/STRIDE groups of STRIDE lanes).  STRIDE = 64 is a no-op.
template <int STRIDE>
__device__ __forceinline__ float across_groups_max(float v) {
  if constexpr (STRIDE <= 8) v = vmax(v, dpp<kDppRor8>(v));
  if constexpr (STRIDE <= 16) { const f32x2 r = pair_xor16(v); v = vmax(r[0], r[1]); }
  if constexpr (STRIDE <= 32) { const f32x2 r = pair_xor32(v); v = vmax(r[0], r[1]); }
  return v;
}

template <int STRIDE>
__device__ __forceinline__ float across_groups_sum(float v) {
  // Every lane of an exchanged pair adds the same two operands.
  if constexpr (STRIDE <= 8) v += dpp<kDppRor8>(v);
  if constexpr (STRIDE <= 16) { const f32x2 r = pair_xor16(v); v = r[0] + r[1]; }
  if constexpr (STRIDE <= 32) { const f32x2 r = pair_xor32(v); v = r[0] + r[1]; }
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- Explicit memory pipelining ------------------------------------------
// s_waitcnt vmcnt(N): at most N vector-memory operations of this wavefront
// still outstanding (loads complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// One direct-to-LDS load of 1 KB: lane i's 16 bytes at src land at dst + 16 i
// (dst is the same for the whole wavefront).
__device__ __forceinline__ void dma16(const void *src, char *dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)dst, 16, 0, 0);
}
// The same with the non-temporal cache policy (data streamed once).
__device__ __forceinline__ void dma16_nt(const void *src, char *dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)dst, 16, 0, 2);
}

// MFMA operand reads from LDS, issued as inline assembly: the compiler does
// not associate them with the direct-to-LDS loads (whose completion the
// kernels await themselves), keeps them in program order with the other
// volatile statements, and leaves their completion to an explicit lgkmcnt
// wait.  Addresses are LDS byte addresses.
template <int OFF>
__device__ __forceinline__ u32x4 lds_b128(uint32_t addr) {
  u32x4 v;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF) : "memory");
  return v;
}
// Transposing read (ds_read_b64_tr_b16): in each group of 16 lanes, lane i
// receives element j from lane 4j + i/4, element i mod 4 of that lane's 8 bytes.
template <int OFF>
__device__ __forceinline__ u32x2 lds_tr16(uint32_t addr) {
  u32x2 v;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF) : "memory");
  return v;
}

// Calls f(integral_constant<int, i>) for i = 0, 1, ... in order.
template <int... is, class F>
__device__ __forceinline__ void for_each_index(std::integer_sequence<int, is...>, F &&f) {
  (f(std::integral_constant<int, is>{}), ...);
}

// Two fp32 values -> the element type's packed pair (round to nearest even).
template <class E>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  if constexpr (__is_same(typename E::storage, _Float16)) return pack_f16(a, b);
  else return pack_bf16(a, b);
}

}  // namespace pa
