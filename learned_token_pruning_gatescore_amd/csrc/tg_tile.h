// tg_tile.h -- LDS tiles of 32 rows x D bf16 for the attention kernels:
// layout, direct-load offsets and MFMA 32x32x16 fragment reads.
#pragma once

#include "tg_common.h"

namespace tg {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int AB_T = 32;   // rows per streamed tile
constexpr int AB_NW = 8;   // waves per work-group (two per SIMD)

// LDS layout of a 32-row bf16 tile: chunk-major.  Chunk c (16 bytes = 8
// elements of every row) is a 512-byte block of 32 rows; row r sits in slot
// r ^ 4 (c % 4) of it.  One 1 KB direct load fills two chunks of all 32 rows.
// Both fragment reads are conflict-free and every fragment address is a
// per-lane base plus a compile-time offset:
//   row reads (ds_read_b128, k = column): 16 lanes read 16 rows of one chunk,
//     16 distinct slots of the 256-byte bank window;
//   transposing reads (ds_read_b64_tr_b16, k = row): 32 lanes read 4
//     consecutive rows of 4 chunks c with distinct c % 4; the XOR moves the
//     four chunks' rows to distinct slots.
template <int D>
struct BTile {
  static constexpr int C = D / 8;        // 16-byte chunks per row
  static constexpr int NI = C / 2;       // 1 KB direct loads per tile
  static constexpr int TILE = AB_T * D;  // u16 per tile
  static constexpr int NKS = D / 16, NDB = D / 32;
  // byte offset in global memory of the 16 bytes that lane fills in direct
  // load i of a tile (row stride rs bytes)
  __device__ static uint32_t goff(int i, int lane, uint32_t rs) {
    const int c = 2 * i + (lane >> 5), row = (lane & 31) ^ (4 * (c & 3));
    return (uint32_t)row * rs + (uint32_t)c * 16u;
  }
};

// Per-lane fragment bases into a tile (MFMA 32x32x16 operand layouts).
template <int D>
struct BFrag {
  using T = BTile<D>;
  int rb[2];  // row read, even / odd k-step
  int tb[2];  // transposing read rr
  __device__ void init(int lane) {
    const int l32 = lane & 31, hl = lane >> 5;
#pragma unroll
    for (int par = 0; par < 2; ++par) rb[par] = hl * 256 + ((l32 ^ (8 * par + 4 * hl)) * 8);
    const int gi = lane >> 4, li = lane & 15, kq = li >> 2, cc = li & 3;
    const int cl = 2 * (gi & 1) + (cc >> 1);  // chunk % 4
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) tb[rr] = cl * 256 + (4 * ((hl + 2 * rr) ^ cl) + kq) * 8 + 4 * (cc & 1);
  }
  // A (or B) operand, k = column: lane holds row l32, columns 16 ks + 8 hl .. +8
  __device__ __forceinline__ u32x4 rows(const uint16_t *t, int ks) const {
    return *(const u32x4 *)(t + rb[ks & 1] + 512 * ks);
  }
  // A operand, k = row: lane holds column 32 db + l32 of rows 16 hf + 8 (e / 4) + 4 hl + e % 4
  // (slot e), matching register 8 hf + e of a 32x32 accumulator whose rows are the tile rows
  __device__ __forceinline__ u32x4 tr(const uint16_t *t, int hf, int db) const {
    const u32x2 lo = __builtin_bit_cast(
        u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(t + tb[0] + 1024 * db + 128 * hf)));
    const u32x2 hi = __builtin_bit_cast(
        u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(t + tb[1] + 1024 * db + 128 * hf)));
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  }
};

// 16-deep operand that adds x (split into three bf16 parts, k = 0, 1, 2) to
// every product of its row (A side) or column (B side), against kOnes.
__device__ __forceinline__ u32x4 aug3(float x, int hl) {
  const uint32_t h = f32_to_bf16_bits(x);
  const float r1 = x - bf16_lo(h);
  const uint32_t m = f32_to_bf16_bits(r1);
  const uint32_t l = f32_to_bf16_bits(r1 - bf16_lo(m));
  return hl == 0 ? u32x4{h | (m << 16), l, 0u, 0u} : u32x4{0u, 0u, 0u, 0u};
}
__device__ __forceinline__ u32x4 ones3(int hl) {
  return hl == 0 ? u32x4{0x3F803F80u, 0x00003F80u, 0u, 0u} : u32x4{0u, 0u, 0u, 0u};
}

}  // namespace tg
