// Device helpers shared by the forward kernels (fa_fwd.hip) and the MFMA
// backward kernels (fa_bwd.hip): vector types, the two 16-bit input types,
// the K/V tile geometry with its LDS swizzles, and the HBM -> LDS copy.
// Not installed; callers use include/fa.h.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// The two 16-bit input types of the MFMA kernel. P is rounded to the input
// type for the PV product; its row-sum bound (the rescale trigger of the
// softmax below) keeps every P inside that type's range.
template <typename E>
struct Elt;
template <>
struct Elt<__bf16> {
  typedef __bf16 x8 __attribute__((ext_vector_type(8)));
  typedef __bf16 x4 __attribute__((ext_vector_type(4)));
  typedef __bf16 x2 __attribute__((ext_vector_type(2)));
  static constexpr float kRowSumLimit = 1.8446744e19f;   // 2^64
  static __device__ __forceinline__ f32x16 mfma(x8 a, x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ float dot2(x2 a, x2 b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
  }
};
template <>
struct Elt<_Float16> {
  typedef _Float16 x8 __attribute__((ext_vector_type(8)));
  typedef _Float16 x4 __attribute__((ext_vector_type(4)));
  typedef _Float16 x2 __attribute__((ext_vector_type(2)));
  // 2^15: a lane's row sum bounds each of its P values, so every P stays
  // below the float16 maximum (65504) between rescales.
  static constexpr float kRowSumLimit = 32768.f;
  static __device__ __forceinline__ f32x16 mfma(x8 a, x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ float dot2(x2 a, x2 b, float c) {
    return __builtin_amdgcn_fdot2(a, b, c, false);
  }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ================================================= 16-bit inputs (bf16, fp16)
// S^T tile = K Q^T with v_mfma_f32_32x32x16_bf16 (or _f16): A = 32 keys x 16 dims from
// LDS, B = 16 dims x 32 query rows from registers. In the accumulator, lane
// (q = lane % 32, g = lane / 32) holds rows 8(v/4) + 4g + v%4 of S^T. Loading
// A row r from key pi(r) (bits 2 and 3 of r swapped) makes element v of that
// lane hold key 16(v/8) + 8g + v%8: eight consecutive keys per lane half,
// which is exactly the k-slot order the PV MFMA wants for its B operand.
//
// K and V tiles are copied HBM -> LDS by the buffer unit (buffer_load_dwordx4
// ... lds): no VGPRs and no VALU work, and rows past the end of the key axis
// come back as zeros from the buffer range check. Both tiles stay row-major
// ([key][dim]) with a 16-byte-chunk XOR swizzle. The PV MFMA needs V^T as its
// A operand (eight consecutive keys of one dim per lane); ds_read_b64_tr_b16
// delivers exactly that from the row-major V tile: within each 16-lane block,
// lane 4r + c reads 4 dims of key row r and the hardware hands lane j the
// 4 keys of dim j.
__device__ __forceinline__ int perm_row(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// Swizzle modes of a tile copy (Bf16Tile::swz).
constexpr int kSwzK = 0, kSwzV = 1, kSwzB = 2;

template <int D, int BN>
struct Bf16Tile {
  static constexpr int DC = D / 16;      // k-steps of the S MFMA
  static constexpr int DB = D / 32;      // 32-dim blocks of the O^T accumulator
  static constexpr int KB = BN / 32;     // 32-key blocks of S^T
  static constexpr int KC = BN / 16;     // 16-key chunks of the PV MFMA
  static constexpr int ROW = D * 2;      // bytes per K or V row in LDS
  static constexpr int CPR = D / 8;      // 16-byte chunks per row
  static constexpr int TILE = BN * ROW;  // bytes per K or V tile
  static constexpr int STAGE = 2 * TILE;
  static constexpr int NI = BN * CPR / 64;       // 1 KB DMA wave-instructions per tile
  static constexpr int NIW = NI / 4;             // ... per wavefront
  static_assert(NI % 4 == 0, "each wavefront issues the same number of DMA instructions");

  // Swizzles (XOR on a row's 16-byte chunk index), by read pattern:
  // K reads: 16 lanes read one chunk of 16 different keys -> XOR with the key.
  static constexpr int swz_k(int key) { return CPR >= 16 ? (key & 15) : ((key >> 1) & 7); }
  // V transpose reads: 32 lanes read 4 chunks of 4 consecutive keys -> move
  // each key of the group of 4 to its own group of 4 chunks.
  static constexpr int swz_v(int key) { return CPR >= 16 ? 4 * (key & 3) : 4 * ((key >> 1) & 1); }
  // Both patterns on one copy: a bit permutation of the row bits that the
  // row reads need distinct (CPR >= 16: the low four bits, their two halves
  // swapped; CPR = 8, two rows per 256 bytes: bits 1-3, bit 1 moved to the
  // top). Any bijection of those bits serves the row reads; these also put
  // the rows of a transposed read on different chunk groups. Rows r and r + 4
  // differ by 1 in the XOR when r % 8 < 4 (bit 2 of r is 0).
  static constexpr int swz_b(int key) {
    return CPR >= 16 ? ((key & 3) << 2) | ((key >> 2) & 3) : (((key >> 1) & 1) << 2) | ((key >> 2) & 3);
  }
  static constexpr int swz(int key, int mode) {
    return mode == kSwzK ? swz_k(key) : mode == kSwzV ? swz_v(key) : swz_b(key);
  }
  // Tile byte offset that LDS chunk P of a copy reads: logical chunk
  // (P % CPR) ^ swz(row) of row P / CPR.
  static constexpr int chunk_off(int P, int mode) { return ((P % CPR) ^ swz(P / CPR, mode)) << 4; }
  static constexpr int dma_off(int P, int mode) { return (P / CPR) * ROW + chunk_off(P, mode); }
  // The offsets of copy instruction k (chunks 64k.. of a wavefront's share)
  // differ from those of instruction 0 by the same XOR in every lane: the row
  // step and the swizzle touch disjoint bits (checked below). One register
  // per buffer then holds a lane's offsets.
  static constexpr int dma_xor(int k, int mode) { return dma_off(64 * k, mode) ^ dma_off(0, mode); }
  static constexpr bool xor_property(int mode) {
    for (int k = 0; k < NI; ++k)
      for (int lane = 0; lane < 64; ++lane)
        if ((dma_off(64 * k + lane, mode) ^ dma_off(lane, mode)) != dma_xor(k, mode)) return false;
    return true;
  }

  // Strided rows (a row stride R that is a multiple of ROW): the row part of
  // an offset, row * R, no longer fits the XOR. It is additive instead
  // (instruction k adds k * RPI * R, uniform) and stays in the vector offset,
  // which the buffer range check covers; the chunk part keeps its
  // per-instruction XOR.
  static constexpr int RPI = 64 / CPR;                   // rows per copy instruction
  static constexpr int chunk_xor(int k, int mode) { return dma_xor(k, mode) & (ROW - 1); }
};

// The XOR property of the copy offsets for every tile shape the kernels use.
template <int D, int BN>
constexpr bool tile_offsets_by_xor() {
  using T = Bf16Tile<D, BN>;
  return T::xor_property(kSwzK) && T::xor_property(kSwzV) && T::xor_property(kSwzB) &&
         T::swz_b(4) == 1;
}
static_assert(tile_offsets_by_xor<64, 64>() && tile_offsets_by_xor<128, 32>() &&
                  tile_offsets_by_xor<256, 32>() && tile_offsets_by_xor<64, 32>() &&
                  tile_offsets_by_xor<128, 64>(),
              "copy offsets of instruction k: instruction 0's XOR a lane-independent constant");

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

template <typename X8>
__device__ __forceinline__ X8 read_v_pair(const char* base, int off0, int off1) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(lds_char*)(base + off0));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(lds_char*)(base + off1));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(X8, v);
}

// One 16-byte-per-lane HBM -> LDS copy: lane l's 16 bytes at base + voff land
// at lds + 16 l (bytes past `bytes` read as zero).
__device__ __forceinline__ void dma16(const void* base, unsigned bytes, int voff, char* lds) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_char*)lds, 16, voff, 0, 0, 0);
}

__device__ __forceinline__ void wait_dma_and_sync() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

}  // namespace fa
