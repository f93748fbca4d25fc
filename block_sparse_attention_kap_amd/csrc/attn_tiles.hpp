// bf16 tile machinery shared by the attention kernels: swizzled HBM -> LDS tile
// copies, the transposed LDS read and the walk-position encoding.
#pragma once

#include "cosa_common.hpp"

#define COSA_MAX_NB 4096  // largest number of blocks per sequence (host-validated)

namespace cosa {

// K and V tiles are copied HBM -> LDS with global_load_lds (16 bytes per lane, no
// register staging).  Each LDS row of 16-byte chunks is XOR-swizzled so that the
// MFMA operand reads are free of bank conflicts (swz_k, swz_v below).  The V operand
// of P.V is read with ds_read_b64_tr_b16: a 16-lane group pointing at a 4 x 16
// block (lane s -> row s/4, columns 4 (s%4) .. +3) receives one column per lane,
// i.e. four consecutive keys of one head dimension, which is exactly the MFMA A
// fragment of V^T.
// NTH threads share the copies of a tile: one query block's waves (BLK / 32 of them), or
// the waves of several query heads that walk one list.
template <int BLK, int D, int NTH = BLK * 2>
struct Tile2 {
  static constexpr int NW = BLK / 32;                 // waves per query block
  static constexpr int NT = NTH;
  static constexpr int CPR = D / 8;                   // 16-byte chunks per row
  static constexpr int LOADS = BLK * CPR / NT;        // copies per thread per tile
  static_assert(BLK * CPR % NT == 0 && NT % CPR == 0, "tile copy shape");
};

// 16-byte chunk c of LDS row r sits at position c ^ swz(r).  With 64 banks of 4 bytes,
// a 256-byte row (D = 128) spans every bank once and a 128-byte row (D = 64) half of
// them.  K: the 16 lanes of a b128 read cover 16 consecutive rows at one chunk.  V: a
// 32-lane transposed read covers 4 consecutive rows x 4 consecutive chunks.
template <int D>
__device__ __forceinline__ int swz_k(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int swz_v(int row) {
  return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
}

// Buffer resource for raw buffer copies on gfx9: base, stride 0, byte range, and
// the gfx9 default word 3.  Reads past the range return zeros instead of faulting.
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
__device__ void raw_buffer_load_lds(i32x4 rsrc, __attribute__((address_space(3))) uint32_t* lds,
                                    int size, int voffset, int soffset, int offset,
                                    int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");

__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu));
  r[2] = (int)bytes;
  r[3] = 0x00020000;
  return r;
}

// Copy one BLK x D bf16 tile (row-major, swizzled) from HBM into LDS.  The buffer
// descriptor covers the whole head (loop-invariant); the tile's byte offset and copy
// `it`'s RPI-row step go through the scalar offset, and each lane keeps one
// loop-invariant byte offset, so the copies cost one VGPR and no 64-bit arithmetic.
template <int BLK, int D, bool VSW, int NTH = BLK * 2>
__device__ __forceinline__ void issue_tile(const i32x4 rs, int tile_off, bf16_t* lds, int tid,
                                           int wave_base) {
  typedef Tile2<BLK, D, NTH> TT;
  constexpr int RPI = TT::NT / TT::CPR;
  const int rl = tid / TT::CPR;
  const int pos = tid % TT::CPR;
#pragma unroll
  for (int it = 0; it < TT::LOADS; ++it) {
    const int row = it * RPI + rl;
    const int c = pos ^ (VSW ? swz_v<D>(row) : swz_k<D>(row));
    const int voff = (rl * D + c * 8) * 2;
    bf16_t* dst = lds + (it * TT::NT + wave_base) * 8;  // wave-uniform 1 KB slab
    raw_buffer_load_lds(rs, (__attribute__((address_space(3))) uint32_t*)dst, 16, voff,
                        tile_off + it * RPI * D * 2, 0, 0);
  }
}

__device__ __forceinline__ void wait_copies() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), other counters untouched
}

__device__ __forceinline__ bf16x4 read_tr(const bf16_t* p) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)p);
  return __builtin_bit_cast(bf16x4, r);
}

// A walk position is encoded as its physical page | DIAG_BIT when the block is the
// diagonal one | TAIL_BIT when it is a ragged last block; STOP ends the walk.
constexpr int DIAG_BIT = 0x8000;
constexpr int TAIL_BIT = 0x4000;   // the ragged last block of the sequence
constexpr int PAGE_MASK = 0x0FFF;  // pages < COSA_MAX_NB
constexpr int STOP = 0xFFFF;

}  // namespace cosa
