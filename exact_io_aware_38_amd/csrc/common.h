// Device-side building blocks shared by the attention kernels (gfx950 only).
//
// Lane layouts used throughout (checked on the hardware with an in-bounds
// probe of the builtins):
//  * v_mfma_f32_32x32x16_bf16: A operand lane l holds row (l % 32) and the 8
//    reduction slots 8*(l/32) .. 8*(l/32)+7; B operand lane l holds column
//    (l % 32) and the same 8 slots; accumulator register i of lane l holds
//    row 8*(i/4) + 4*(l/32) + (i%4), column (l % 32).
//  * ds_read_b64_tr_b16: within each 16-lane group, lane L supplies the
//    address of 4 consecutive 16-bit elements of row r0 + L/4, columns
//    c0 + 4*(L%4) .. +3 of a row-major LDS matrix; lane j of the group then
//    receives the 4 elements of rows r0 .. r0+3 in column c0 + j.
//  * permlane32_swap(x, x) returns {x[l % 32], x[l % 32 + 32]} in every lane.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace attn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 2^x on the transcendental unit; 2^-inf = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 2^x on the FMA pipe, the software exponential of "Flash Attention FA1->FA4 /
// pre-training practice" section 2.3: 2^x = 2^n 2^f, n = floor(x), f in
// [0, 1), 2^f by a cubic fitted to it on [0, 1) (relative error at most
// 8.6e-5, below a bf16 rounding step), 2^n by an exponent add. Arguments
// below -127 give 0, as exp2 does in the range the softmax uses.
__device__ __forceinline__ float poly_exp2(float x) {
  x = fmaxf(x, -127.f);
  const float n = __builtin_floorf(x);
  const float f = x - n;
  float p = __builtin_fmaf(f, 0.07706520f, 0.22764701f);
  p = __builtin_fmaf(f, p, 0.69511634f);
  p = __builtin_fmaf(f, p, 1.0f);
  const float r = __builtin_ldexpf(p, (int)n);
  return x <= -127.f ? 0.f : r;
}

// max of x over lanes l and l^32.
__device__ __forceinline__ float max_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// sum of x over lanes l and l^32.
__device__ __forceinline__ float sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

// Transposed 8-byte LDS read (see the layout note at the top of this file).
__device__ __forceinline__ bf16x4 lds_read_tr(const bf16* p) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  return __builtin_bit_cast(bf16x4, r);
}

__device__ __forceinline__ bf16x8 cat4(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Round-to-nearest-even float -> bf16 of 8 values.
__device__ __forceinline__ bf16x8 to_bf16x8(float a0, float a1, float a2, float a3,
                                            float a4, float a5, float a6, float a7) {
  bf16x8 r;
  r[0] = (bf16)a0; r[1] = (bf16)a1; r[2] = (bf16)a2; r[3] = (bf16)a3;
  r[4] = (bf16)a4; r[5] = (bf16)a5; r[6] = (bf16)a6; r[7] = (bf16)a7;
  return r;
}

// Max and sum of 32 values as balanced trees (max3 where possible), so that
// the reductions do not form long dependency chains.
__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

__device__ __forceinline__ float tree_max32(const float* v) {
  float t[11];
#pragma unroll
  for (int i = 0; i < 10; ++i) t[i] = max3f(v[3 * i], v[3 * i + 1], v[3 * i + 2]);
  t[10] = fmaxf(v[30], v[31]);
  const float u0 = max3f(t[0], t[1], t[2]), u1 = max3f(t[3], t[4], t[5]);
  const float u2 = max3f(t[6], t[7], t[8]), u3 = fmaxf(t[9], t[10]);
  return fmaxf(max3f(u0, u1, u2), u3);
}

__device__ __forceinline__ float tree_sum32(const float* v) {
  float t[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) t[i] = v[2 * i] + v[2 * i + 1];
#pragma unroll
  for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
    for (int i = 0; i < w; ++i) t[i] = t[2 * i] + t[2 * i + 1];
  return t[0];
}

// LDS tiles of 32 or 64 rows x D bf16 are stored unpadded, with the 16-byte chunks
// of each row XOR-permuted by this row function. gfx950 LDS serves 256 bytes
// per clock over 64 banks: 16-byte row reads (16 consecutive rows, same
// logical chunk) and transposed 8-byte reads (4 consecutive rows x 4 adjacent
// chunks per 32 lanes) then both hit 16 distinct 16-byte bank groups, which a
// conflict-counter probe of every read pattern used here confirmed.
template <int D>
__device__ __forceinline__ int chunk_swizzle(int row) {
  if constexpr (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
  else return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

// Workgroup order: the hardware hands consecutive workgroup ids to the 8 XCDs
// in turn, each with its own L2. Renumber so that each XCD receives a
// contiguous range of logical ids, i.e. all tiles of a few heads, which then
// share K/V lines in that XCD's L2.
__device__ __forceinline__ int xcd_logical_id(int linear, int total) {
  if ((total & 7) != 0) return linear;
  return (linear & 7) * (total >> 3) + (linear >> 3);
}

// Workgroup -> (tile, unit) for grids of `tiles` tiles per unit (a unit being
// a head, or a group of heads) whose tiles differ in length, tile 0 the
// longest. Each XCD receives a contiguous range of logical ids (whole units
// when the range holds whole units, so the units' K/V lines stay in that XCD's
// L2), and inside the range the tile index varies slowest: the XCD starts the
// longest tiles of its units first, which keeps the short ones for the end of
// the launch. When the range holds a multiple of 4 units, it is taken 4 units
// at a time (longest tiles of units 0-3 first, then of units 4-7, ...): more
// workgroups of one unit then stream its K/V lines together, which halves the
// L2 misses of an XCD holding 8 heads at no cost in balance.
__device__ __forceinline__ void xcd_tile_order(int total, int tiles, int& tile, int& unit) {
  const int W = xcd_logical_id(blockIdx.x, total);
  if ((total & 7) == 0) {
    const int R = total >> 3;
    if (R % tiles == 0) {
      const int nu = R / tiles;
      const int G = (nu % 4 == 0) ? 4 : nu;     // units taken together
      const int x = W / R, s = W % R;
      const int grp = s / (G * tiles), r = s % (G * tiles);
      tile = r / G;
      unit = x * nu + grp * G + r % G;
      return;
    }
  }
  tile = W % tiles;
  unit = W / tiles;
}

// Philox4x32-10, the counter-based generator of Salmon, Moraes, Dror and Shaw
// ("Parallel random numbers: as easy as 1, 2, 3", SC 2011): ten rounds of two
// 32x32->64-bit products whose halves are mixed with the other two counter
// words and the key; the key advances by the two Weyl constants between
// rounds. Returns the four output words.
__host__ __device__ inline u32x4 philox4x32_10(u32x4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
    u32x4 n;
    n[0] = (uint32_t)(p1 >> 32) ^ c[1] ^ k0;
    n[1] = (uint32_t)p1;
    n[2] = (uint32_t)(p0 >> 32) ^ c[3] ^ k1;
    n[3] = (uint32_t)p0;
    c = n;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

// The dropout bytes of one 4x4 block of the score matrix of query head bh
// (= b * Hq + h): query rows 4 i4 .. 4 i4 + 3, keys 4 j4 .. 4 j4 + 3 (positions
// within the sequence). Word w holds query row 4 i4 + w; byte t of it key
// 4 j4 + t. Counter (j4, i4, bh, offset), key the 64-bit seed.
__host__ __device__ inline u32x4 dropout_block(const DropParams& dp, uint32_t i4, uint32_t j4, uint32_t bh) {
  u32x4 c;
  c[0] = j4;
  c[1] = i4;
  c[2] = bh;
  c[3] = dp.offset;
  return philox4x32_10(c, dp.seed_lo, dp.seed_hi);
}

// Table parameter of a kernel launched on one dense problem.
struct NoTable {};

// Where this workgroup sits in a packed launch: the sequence, the unit (head
// or group of heads) and the tile rank inside the unit (0 first). Wave-uniform;
// a binary search over the table's workgroup offsets.
struct SeqCoord {
  int seq, unit, t;
};
__host__ __device__ inline SeqCoord seq_coord_of(const SeqTable& T, int id) {
  int x = 0, r = id, per = T.units;
  if (T.split8) {
    x = id & 7;
    r = id >> 3;
    per = T.units >> 3;
  }
  int s = 0;
#pragma unroll
  for (int step = SEQ_MAX / 2; step > 0; step >>= 1)
    if (s + step < T.n && T.wg0[s + step] <= r) s += step;
  const int local = r - T.wg0[s];
  return SeqCoord{s, x * per + local % per, local / per};
}
__device__ __forceinline__ SeqCoord seq_coord(const SeqTable& T) { return seq_coord_of(T, blockIdx.x); }

}  // namespace attn
