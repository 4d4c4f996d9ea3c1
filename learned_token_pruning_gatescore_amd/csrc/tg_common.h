// tg_common.h -- device-side helpers shared by the libtokengate kernels
// (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// bf16 <-> fp32.  Storage is raw uint16; widening is exact, narrowing rounds
// to nearest even (NaN kept quiet).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 pair (lo in the low half), round to nearest even
// (one v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2_t));
}

// ---------------------------------------------------------------------------
// Matrix-core products (layouts measured on gfx950):
//   32x32x16: A[i][k] in lane i + 32*(k/8), element k%8;  B[k][j] in lane
//             j + 32*(k/8), element k%8;  C[i][j] in lane j + 32*((i/4)%2),
//             register (i/8)*4 + i%4.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x16 mfma32(const u32x4 &a, const u32x4 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Row of the 32x32 accumulator held in register r by a lane in half hl (= lane / 32).
__device__ __forceinline__ constexpr int acc_row(int r, int hl) { return 8 * (r >> 2) + 4 * hl + (r & 3); }

__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// ---------------------------------------------------------------------------
// Direct buffer -> LDS loads.  Lane l's bytes land at lds + l * size; offsets
// past the resource's num_records read as zero.  They are issued through
// inline assembly so that the compiler does not track them: it would
// otherwise wait for every load in flight before each LDS read of ANY buffer
// (it cannot tell the ring stages apart), which drains the prefetch pipeline.
// Callers order them with sync_vm<N>(): wait until at most N vector-memory
// loads of this wave are in flight, then a work-group barrier.
// ---------------------------------------------------------------------------
typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i32x4 buffer_rsrc(const void *base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return i32x4{(int)(uint32_t)a, (int)(uint32_t)(a >> 32), (int)bytes, 0x00020000};
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// A wave-uniform value in scalar registers (the resource, the LDS address and
// soffset must be the same for every lane of the wave).
__device__ __forceinline__ i32x4 uniform(const i32x4 &r) {
  return i32x4{__builtin_amdgcn_readfirstlane(r[0]), __builtin_amdgcn_readfirstlane(r[1]),
               __builtin_amdgcn_readfirstlane(r[2]), __builtin_amdgcn_readfirstlane(r[3])};
}

// lds is an LDS byte address (see lds_addr).
__device__ __forceinline__ void dma_b128(const i32x4 &rsrc, uint32_t lds, uint32_t voffset, uint32_t soffset) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voffset), "s"(uniform(rsrc)),
                  "s"(__builtin_amdgcn_readfirstlane(soffset))
               : "memory", "m0");
}
__device__ __forceinline__ void dma_b32(const i32x4 &rsrc, uint32_t lds, uint32_t voffset, uint32_t soffset) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voffset), "s"(uniform(rsrc)),
                  "s"(__builtin_amdgcn_readfirstlane(soffset))
               : "memory", "m0");
}

// Wait until at most N vector-memory loads of this wave are outstanding and
// every LDS access of this wave has completed, then a work-group barrier.
// Also a compiler barrier for memory operations.
template <int N>
__device__ __forceinline__ void sync_vm() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" :: "n"(N) : "memory");
}

// Consume a loaded value here, so that the compiler waits for its load at
// this point.  The direct buffer->LDS loads above are inline asm the compiler
// does not track; a load of its own that it still counts as in flight at a
// loop header makes it put a full `s_waitcnt vmcnt(0)` inside the loop, which
// at run time also waits for every direct load in flight (the tile
// prefetches), once per iteration.  Settling the prologue's loads before the
// loop keeps that wait out of it.
__device__ __forceinline__ void settle(const u32x4 &x) { asm volatile("" ::"v"(x)); }
__device__ __forceinline__ void settle(float x) { asm volatile("" ::"v"(x)); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

}  // namespace tg
