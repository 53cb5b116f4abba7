// hcgr_device.h -- gfx950 device helpers shared by the kernel sources:
// bf16 packing, the v_mfma_f32_16x16x32_bf16 wrapper, range-limited buffer
// resources and their loads/stores, and the LDS-only barrier. Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hcgr {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf1(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
// float -> bf16, round to nearest even (gfx950 v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  bf16x2_t v;
  v.x = (__bf16)lo;
  v.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t to_bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ __forceinline__ bf16x8_t as_bf8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ __forceinline__ f32x4_t mfma16(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf8(a), as_bf8(b), c, 0, 0, 0);
}
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) uint8_t lds_u8_t;
// Buffer resource over [base, base + bytes): loads past the range return 0
// and stores past it are dropped. Word 3 (0x00020000) is the 32-bit data
// format that gfx9-family raw buffer descriptors use.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// Range of an optional tensor: a NULL base gives an empty range, whose loads
// return 0 and whose stores are dropped (the mix entry point passes no y and
// no R2 output this way).
__device__ __forceinline__ rsrc_t make_rsrc_opt(const uint16_t* base, int64_t off, uint32_t bytes) {
  return base ? make_rsrc(base + off, bytes) : make_rsrc(nullptr, 0u);
}
__device__ __forceinline__ uint4 bld16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ void bst16(rsrc_t r, uint32_t off, uint4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, (int)off, 0, 0);
}
// Non-temporal (streaming) cache policy, for data a kernel reads or writes
// once: R in and R2 out of the combine pass, when R2 is too large for the
// caches to keep it until the up kernel reads it back. Measured on MI355X
// (HC = 4, HS = 2560): the large-token down kernel 17% faster at M = 8192 and
// 65536 with R read and R2 written this way (the whole call 7-9% faster from
// M = 8192), the combine-only kernel 11-20% faster at M = 8192; but the
// staged up kernel 10-20% slower at M = 256 .. 2048, where R2 stays in the
// 256 MB Infinity Cache for it. y (read once per stream) keeps the default.
constexpr int kNonTemporal = 2;
constexpr double kStreamBytes = 256.0 * 1024 * 1024;  // Infinity Cache
__device__ __forceinline__ uint4 bld16_nt(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kNonTemporal));
}
__device__ __forceinline__ void bst16_nt(rsrc_t r, uint32_t off, uint4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, (int)off, 0, kNonTemporal);
}
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 bld8(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
}
__device__ __forceinline__ void bst8(rsrc_t r, uint32_t off, uint2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, v), r, (int)off, 0, 0);
}
// Agent-scope coherent accesses (the SC1 cache-policy bit): stores write
// through the XCD's L2 (the line does not stay dirty there), loads do not
// return a line another XCD may have changed.
constexpr int kAgentCoherent = 16;
// Write-through stores, for a kernel's outputs at decode sizes, where the
// write-back of dirty lines at the kernel's end would otherwise sit on the
// critical path.
__device__ __forceinline__ void bst16_wt(rsrc_t r, uint32_t off, uint4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, (int)off, 0, kAgentCoherent);
}
__device__ __forceinline__ void st_f32(float* p, float v, int wt) {
  if (wt) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // a store with SC1
  else *p = v;
}
// Workgroup barrier that orders LDS traffic only: waits for this wave's LDS
// operations, then s_barrier. Unlike __syncthreads it does not wait for
// outstanding global->LDS loads, which may stay in flight across it (their
// target is read only after an explicit full wait).
__device__ __forceinline__ void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
// logistic function through the hardware 2^x and reciprocal: 1/(1 + 2^(-v*log2 e))
__device__ __forceinline__ float sigmoid_f(float v) { return __builtin_amdgcn_rcpf(1.0f + __expf(-v)); }

}  // namespace hcgr
