// Tile helpers shared by the forward and backward kernels: the LDS DMA
// (global or buffer loads straight into LDS), compile-time loops and the
// register pins the pipelined kernels use.
#pragma once

#include "common.h"

#include <type_traits>
#include <utility>

namespace attn {
namespace {

constexpr int TILE_ROWS = 64;        // sequence rows per staged tile

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

// 16 bytes per lane from global memory straight into LDS at base + 16 * lane
// (base must be wave-uniform). Issued as inline assembly: the compiler would
// otherwise make every later LDS read wait for all outstanding DMA (it cannot
// tell the ring stages apart), which serialises the prefetch; the kernels wait
// for their DMA explicitly (s_waitcnt vmcnt + s_barrier) before reading a stage.
// On this chip generation an LDS DMA instruction must not read M0 in the cycle
// right after a scalar write to it, so every helper puts one s_nop between
// the two (the compiler's hazard pass does not look inside inline assembly).
__device__ __forceinline__ void dma16(const void* g, lds_void* base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)base);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(m0), "v"(g)
               : "memory", "m0");
}

// Wave-uniform 64-bit pointer held in scalar registers.
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t x = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
  return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// Scalar-base forms: lane address = sbase + voff (32-bit unsigned byte
// offset), which keeps the per-lane address arithmetic to 32 bits.
__device__ __forceinline__ void dma16s(const void* sbase, uint32_t voff, lds_void* base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)base);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(m0), "v"(voff), "s"(uniform_ptr(sbase))
               : "memory", "m0");
}
__device__ __forceinline__ void dma4s(const void* sbase, uint32_t voff, lds_void* base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)base);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
               :
               : "s"(m0), "v"(voff), "s"(uniform_ptr(sbase))
               : "memory", "m0");
}


// Buffer resource for raw loads with range checking: a lane whose byte
// offset is >= num_bytes reads zeros. Word 3 selects the 32-bit data format
// (format 0 would read zeros everywhere); stride 0 gives a raw buffer.
__device__ __forceinline__ u32x4 buffer_rsrc(const void* base, uint32_t num_bytes) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  u32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((uint32_t)b);
  r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32) & 0xffffu);
  r[2] = __builtin_amdgcn_readfirstlane(num_bytes);
  r[3] = 0x00020000u;
  return r;
}

// 16 bytes per lane from a buffer (offset voff, range-checked) into LDS at
// base + 16 * lane.
__device__ __forceinline__ void dma16b(u32x4 rsrc, uint32_t voff, lds_void* base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)base);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(m0), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

// Same with the LDS byte address given as a wave-uniform base plus a
// compile-time offset (one scalar add builds M0), and a scalar byte offset
// soff added to the address (not range-checked: only voff is compared with
// the buffer size).
template <uint32_t OFF>
__device__ __forceinline__ void dma16b_at(u32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds_base) {
  asm volatile("s_add_u32 m0, %0, %4\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds_base), "v"(voff), "s"(rsrc), "s"(soff), "i"(OFF)
               : "memory", "m0", "scc");
}
template <uint32_t OFF>
__device__ __forceinline__ void dma4b_at(u32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds_base) {
  asm volatile("s_add_u32 m0, %0, %4\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :
               : "s"(lds_base), "v"(voff), "s"(rsrc), "s"(soff), "i"(OFF)
               : "memory", "m0", "scc");
}

// f(integral_constant<int, I>) for I = 0 .. N-1, in order, with I usable as
// a compile-time constant inside f.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Pins where values are computed: results that are only consumed in the next
// pipeline step would otherwise all be computed in one block just before the
// step boundary (instruction selection places pure arithmetic next to its
// first chained use), instead of interleaved with the MFMAs they should hide
// behind. The empty volatile statement forces them to exist at this point.
__device__ __forceinline__ void pin(float& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(float& x, float& y) { asm volatile("" : "+v"(x), "+v"(y)); }
__device__ __forceinline__ void pin(bf16x8& x) {
  u32x4 w = __builtin_bit_cast(u32x4, x);
  asm volatile("" : "+v"(w));
  x = __builtin_bit_cast(bf16x8, w);
}

// Re-define a value that a global load produced before a loop, so the
// compiler knows no load is pending on it inside the loop (it would otherwise
// wait on the memory counter there, which also waits for DMA in flight). The
// caller's first use after this waits for the load, once.
template <typename T>
__device__ __forceinline__ T settle(T x) {
  static_assert(sizeof(T) % 4 == 0, "32-bit registers");
  if constexpr (sizeof(T) == 4) {
    uint32_t w = __builtin_bit_cast(uint32_t, x);
    asm volatile("" : "+v"(w));
    return __builtin_bit_cast(T, w);
  } else {
    typedef uint32_t words __attribute__((ext_vector_type(sizeof(T) / 4)));
    words w = __builtin_bit_cast(words, x);
    asm volatile("" : "+v"(w));
    return __builtin_bit_cast(T, w);
  }
}

}  // namespace
}  // namespace attn
