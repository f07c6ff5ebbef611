// Device helpers shared by the Infini-attention kernels (gfx950 / CDNA4).
//
// Conventions used across the kernels:
//  * bf16 values travel as raw 16-bit patterns (uint16_t); conversion to float is a
//    shift, conversion from float is round-to-nearest-even (the hardware cvt on gfx950).
//  * MFMA 32x32x16 bf16 (v_mfma_f32_32x32x16_bf16): operand A is 32 rows x 16 k, lane l
//    supplies row (l % 32) and the 8 consecutive k values 8*(l / 32) .. +7; operand B is
//    16 k x 32 columns, lane l supplies column (l % 32) and the same 8 k values.  The
//    32x32 fp32 result has 16 registers per lane: register r of lane l is row
//    8*(r/4) + 4*(l/32) + (r%4), column l % 32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace infini {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_to_f32(uint16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x) << 16);
}
__device__ __forceinline__ float bf16lo_to_f32(uint32_t packed) {  // element 0 of a pair
  return __uint_as_float(packed << 16);
}
__device__ __forceinline__ float bf16hi_to_f32(uint32_t packed) {  // element 1 of a pair
  return __uint_as_float(packed & 0xffff0000u);
}

// float -> bf16 (round to nearest even), as raw bits.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 b = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, b);
}
// Two floats -> one dword holding bf16(a) in the low half and bf16(b) in the high half
// (one v_cvt_pk_bf16_f32).
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2 v = __builtin_convertvector(f32x2{a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, v);
}

// Lane l and lane l ^ 32 combined without LDS (v_permlane32_swap): the swap leaves the
// low half's values in both halves of one register and the high half's in the other.
__device__ __forceinline__ float max_across_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_across_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// acc + lo + hi of a packed bf16 pair (v_dot2 against (1, 1); the products are exact).
__device__ __forceinline__ float add_bf16x2(uint32_t packed, float acc) {
  const bf16x2 one = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, packed), one, acc, false);
}

// sigma(x) = ELU(x) + 1 with alpha = 1: x + 1 for x > 0, exp(x) otherwise.
__device__ __forceinline__ float elu_plus_one(float x) {
  return x > 0.f ? x + 1.f : __builtin_amdgcn_exp2f(x * kLog2e);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Split x into bf16 hi + bf16 lo with hi + lo == x to about 2^-17 relative.
__device__ __forceinline__ void split_bf16(float x, uint16_t& hi, uint16_t& lo) {
  hi = f32_to_bf16(x);
  lo = f32_to_bf16(x - bf16_to_f32(hi));
}

// LDS transpose read (gfx950 ds_read_b64_tr_b16).  Within each group of 16 lanes, lane j
// supplies the address of 4 consecutive 16-bit elements; lane i of the group receives
// element i % 4 of the loads of lanes 4r + i / 4, r = 0..3.  With a row-major [k][n] tile
// and lane j addressing &X[k0 + j/4][n0 + 4*(j%4)], lane i receives X[k0 + r][n0 + i] for
// r = 0..3: four consecutive k of column n0 + i, i.e. half of an MFMA operand slice.
typedef short i16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* lds_ptr) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds_ptr));
  return __builtin_bit_cast(u32x2, r);
}

// The 8 consecutive-k values of a 32x32x16 MFMA operand (A or B) for this lane, from a
// row-major [k][n] bf16 tile in LDS with row pitch `pitch` elements: lane l gets
// X[k0 + 8*(l/32) + 0..7][n0 + l%32].  Two transpose reads.
__device__ __forceinline__ bf16x8 lds_operand_tr(const uint16_t* tile, int pitch, int k0, int n0, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const uint16_t* p = tile + (k0 + 8 * (g >> 1) + (j >> 2)) * pitch + n0 + 16 * (g & 1) + 4 * (j & 3);
  const u32x2 lo = lds_read_tr16(p);
  const u32x2 hi = lds_read_tr16(p + 4 * pitch);
  return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
}

// Raw buffer access: a 128-bit resource (base, size in bytes) built in scalar registers.
// Loads at byte offsets at or beyond `bytes` return zeros, so a tile that runs past the
// end of a segment needs no branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(bytes),
                                           0x00020000);
}
__device__ __forceinline__ u32x4 buffer_ld16(__amdgpu_buffer_rsrc_t r, uint32_t voffset) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(voffset), 0, 0));
}
__device__ __forceinline__ u32x2 buffer_ld8(__amdgpu_buffer_rsrc_t r, uint32_t voffset) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, static_cast<int>(voffset), 0, 0));
}
// Stores at byte offsets at or beyond the resource's `bytes` are dropped.
__device__ __forceinline__ void buffer_st16(__amdgpu_buffer_rsrc_t r, uint32_t voffset, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, static_cast<int>(voffset), 0, 0);
}
// Device-coherent forms (cache policy SC1: the access is performed at device scope, so a
// store is visible to every XCD once it has completed, and a load does not return a line
// another XCD's L2 may hold stale).  For data one workgroup hands to another inside a launch.
constexpr int kCpolDevice = 16;
__device__ __forceinline__ void buffer_st16_dev(__amdgpu_buffer_rsrc_t r, uint32_t voffset, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, static_cast<int>(voffset), 0, kCpolDevice);
}
__device__ __forceinline__ u32x4 buffer_ld16_dev(__amdgpu_buffer_rsrc_t r, uint32_t voffset) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(voffset), 0, kCpolDevice));
}
__device__ __forceinline__ void buffer_st8_dev(__amdgpu_buffer_rsrc_t r, uint32_t voffset, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, static_cast<int>(voffset), 0, kCpolDevice);
}
__device__ __forceinline__ u32x2 buffer_ld8_dev(__amdgpu_buffer_rsrc_t r, uint32_t voffset) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, static_cast<int>(voffset), 0, kCpolDevice));
}
__device__ __forceinline__ void buffer_st4_dev(__amdgpu_buffer_rsrc_t r, uint32_t voffset, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, static_cast<int>(voffset), 0, kCpolDevice);
}
__device__ __forceinline__ float buffer_ld4_dev(__amdgpu_buffer_rsrc_t r, uint32_t voffset) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(voffset), 0, kCpolDevice));
}

// Buffer -> LDS copy of 16 bytes per lane (gfx950): lane i's bytes land at lds_base + 16 i
// (lds_base wave-uniform); offsets past the resource end write zeros.
__device__ __forceinline__ void buffer_to_lds16(__amdgpu_buffer_rsrc_t r, void* lds_base, uint32_t voffset) {
  typedef __attribute__((address_space(3))) void lds_void;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(lds_base), 16, static_cast<int>(voffset), 0, 0, 0);
}

// s_waitcnt with vmcnt <= vm and lgkmcnt = 0 (expcnt not waited on); gfx9 encoding.
template <int VM>
__device__ __forceinline__ void wait_vm_lgkm0() {
  __builtin_amdgcn_s_waitcnt((VM & 15) | (7 << 4) | (0 << 8) | ((VM >> 4) << 14));
}
__device__ __forceinline__ void wait_vm_le(int vm) {   // vm wave-uniform, 0 .. 16
  switch (vm) {
    case 0: wait_vm_lgkm0<0>(); break;
    case 1: wait_vm_lgkm0<1>(); break;
    case 2: wait_vm_lgkm0<2>(); break;
    case 3: wait_vm_lgkm0<3>(); break;
    case 4: wait_vm_lgkm0<4>(); break;
    case 5: wait_vm_lgkm0<5>(); break;
    case 6: wait_vm_lgkm0<6>(); break;
    case 7: wait_vm_lgkm0<7>(); break;
    case 8: wait_vm_lgkm0<8>(); break;
    case 9: wait_vm_lgkm0<9>(); break;
    case 10: wait_vm_lgkm0<10>(); break;
    case 11: wait_vm_lgkm0<11>(); break;
    case 12: wait_vm_lgkm0<12>(); break;
    case 13: wait_vm_lgkm0<13>(); break;
    case 14: wait_vm_lgkm0<14>(); break;
    case 15: wait_vm_lgkm0<15>(); break;
    case 16: wait_vm_lgkm0<16>(); break;
    default: wait_vm_lgkm0<0>(); break;   // anything else: wait for everything
  }
}

// Buffer -> LDS copy of 16 bytes per lane (lane i to lds + 16 i; offsets at or past
// `bytes` read zeros), issued as inline assembly so that the compiler adds no waits of its
// own for it: the kernel orders copies and LDS reads itself, with explicit vmcnt waits
// and barriers.  (The compiler's tracking of the builtin form loses which buffer a copy
// writes across the unrolled pipeline and then holds every operand read until all copies
// in flight have landed.)  M0 must be written one wait state before the copy.
// (Kernels that use it keep no value of their own in M0 and do not mix it with the builtin
// form, so clobbering M0 is safe.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void copy_to_lds(const void* src, uint32_t bytes, const uint16_t* lds, uint32_t voffset) {
  typedef __attribute__((address_space(3))) const uint16_t lds_u16;
  // every operand is wave-uniform; readfirstlane states it, so that they stay in SGPRs
  const uint32_t m0 = static_cast<uint32_t>(
      __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_u16*)lds))));
  const uint64_t a = reinterpret_cast<uint64_t>(src);
  const u32x4 rsrc = {static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a))),
                      static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32) & 0xffffu)),
                      static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(bytes)), 0x00020000u};
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(m0), "v"(voffset), "s"(rsrc)
               : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ u32x2 ld8(const void* p) { return *reinterpret_cast<const u32x2*>(p); }
__device__ __forceinline__ void st8(void* p, u32x2 v) { *reinterpret_cast<u32x2*>(p) = v; }

}  // namespace infini
