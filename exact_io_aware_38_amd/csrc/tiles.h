// Tile helpers shared by the forward and backward kernels: the LDS DMA
// (buffer loads straight into LDS), compile-time loops and the register pins
// the pipelined kernels use.
#pragma once

#include "common.h"

#include <type_traits>
#include <utility>

namespace attn {
namespace {

constexpr int TILE_ROWS = 64;        // the backward pads Sq to a multiple of this

// Buffer resource for raw loads with range checking: a lane whose byte
// offset is >= num_bytes reads zeros. Word 3 selects the 32-bit data format
// (format 0 would read zeros everywhere); stride 0 gives a raw buffer.
// A wave-uniform pointer moved into scalar registers once, so that address
// arithmetic on it stays scalar (the compiler can keep uniform values in
// vector registers, and every buffer descriptor built from one then needs a
// vector add and two readfirstlane per use).
template <typename T>
__device__ __forceinline__ T* wave_uniform(T* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  // readfirstlane returns int: widen each half as unsigned (a sign-extended
  // low half would corrupt the high word)
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (T*)(uintptr_t)((hi << 32) | lo);
}

__device__ __forceinline__ u32x4 buffer_rsrc(const void* base, uint32_t num_bytes) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  u32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((uint32_t)b);
  r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32) & 0xffffu);
  r[2] = __builtin_amdgcn_readfirstlane(num_bytes);
  r[3] = 0x00020000u;
  return r;
}

// LDS DMA: 16 (or 4) bytes per lane from a buffer (byte offset voff,
// range-checked, plus a scalar byte offset soff that is not range-checked)
// straight into LDS at lds_base + OFF + 16 * lane (4 * lane); lds_base must be
// wave-uniform, OFF is a compile-time offset (one scalar add builds M0).
// Issued as inline assembly: the compiler would otherwise make every later
// LDS read wait for all outstanding DMA (it cannot tell the ring slots apart);
// the kernels wait for their DMA explicitly (s_waitcnt vmcnt + s_barrier)
// before reading a slot. On this chip generation an LDS DMA instruction must
// not read M0 in the cycle right after a scalar write to it, hence the s_nop
// (the compiler's hazard pass does not look inside inline assembly).
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
