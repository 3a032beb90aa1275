// tiles_bf16.h - staging of 64-row K/V tiles (D = 128, bf16) through LDS, for workgroups of
// 256 threads. Shared by the hybrid-attention and the state-reduction kernels.
//
// K tile : [64 keys][128 d], rows of 256 B. 16-byte chunk c of row r is stored at chunk
//          c ^ kappa(r & 15). Readers take rows kappa(l%32) + 32*kb at chunk 2s + l/32, so
//          each group of 16 lanes hits 16 distinct chunk columns (no bank conflicts).
// V^T tile: [128 d][64 keys], rows of 128 B: the key index becomes the contiguous MFMA
//          k-dimension. 8-key chunk kc of row d is stored at chunk kc ^ ((d + d/8) & 7):
//          readers (rows d..d+7 at one chunk) and the transposing writers (16 rows at
//          one key) both spread over the bank columns.
#pragma once

#include "common.h"

namespace rehyat {

constexpr int kTileRows = 64;
constexpr int kDim = 128;
constexpr int kKTileBytes = kTileRows * kDim * 2;   // 16 KB
constexpr int kVTileBytes = kTileRows * kDim * 2;   // 16 KB

__device__ __forceinline__ int ktile_off(int r, int c) {
  return r * 256 + ((c ^ kappa(r & 15)) << 4);
}
__device__ __forceinline__ int vtile_off(int d, int key) {
  return d * 128 + ((((key >> 3) ^ ((d + (d >> 3)) & 7))) << 4) + ((key & 7) << 1);
}
// 16-byte chunk kc (keys 8kc..8kc+7) of V^T row d
__device__ __forceinline__ int vtile_chunk_off(int d, int kc) {
  return d * 128 + ((kc ^ ((d + (d >> 3)) & 7)) << 4);
}

__device__ __forceinline__ u32x4 lds_read16(const unsigned char* base, int off) {
  return *reinterpret_cast<const u32x4*>(base + off);
}

// Rows of one tile come from up to two row segments of a [rows, 128] bf16 head:
// tile row w (global window row w0 + w) is segment A row (a_row0 + w) if < na, else
// segment B row (w - na). Rows at or beyond n are zero-filled.
struct RowSrc {
  const uint16_t* a;   // head base of segment A (already offset by the head)
  const uint16_t* b;   // head base of segment B
  int64_t a_row0;
  int64_t na, n;
};

__device__ __forceinline__ const uint16_t* row_ptr(const RowSrc& s, int64_t w) {
  return (w < s.na) ? s.a + (s.a_row0 + w) * kDim : s.b + (w - s.na) * kDim;
}

// Each of 256 threads loads 4 x 16 B of K and of V for tile rows [w0, w0+64).
struct TileRegs {
  u32x4 k[4];
  u32x4 v[4];
};

__device__ __forceinline__ void tile_load(TileRegs& r, const RowSrc& ks, const RowSrc& vs,
                                          int64_t w0, int tid) {
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    int id = it * 256 + tid;
    int row = id >> 4, c = id & 15;
    int64_t w = w0 + row;
    if (w < ks.n) {
      r.k[it] = *reinterpret_cast<const u32x4*>(row_ptr(ks, w) + c * 8);
      r.v[it] = *reinterpret_cast<const u32x4*>(row_ptr(vs, w) + c * 8);
    } else {
      r.k[it] = u32x4{0u, 0u, 0u, 0u};
      r.v[it] = u32x4{0u, 0u, 0u, 0u};
    }
  }
}

__device__ __forceinline__ void tile_store(const TileRegs& r, unsigned char* kt,
                                           unsigned char* vt, int tid) {
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    int id = it * 256 + tid;
    int row = id >> 4, c = id & 15;
    *reinterpret_cast<u32x4*>(kt + ktile_off(row, c)) = r.k[it];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      unsigned w = r.v[it][e >> 1];
      uint16_t h = (e & 1) ? (uint16_t)(w >> 16) : (uint16_t)(w & 0xffffu);
      *reinterpret_cast<uint16_t*>(vt + vtile_off(c * 8 + e, row)) = h;
    }
  }
}

// Transposing fragment read (ds_read_b64_tr_b16) from a row-major bf16 tile with row
// stride `ld` bytes: lane l receives the 8 consecutive rows row0 + 8 (l/32) .. +7 of column
// col0 + (l mod 32), the operand layout of a 32x32x16 MFMA whose contraction runs over
// those rows. Within each 16-lane group lane r addresses row row0 + 8 (group/2) + r/4 at
// columns col0 + 16 (group mod 2) + 4 (r mod 4) .. +3, and lane j of the group receives
// the four rows of column col0 + 16 (group mod 2) + j. With ld = 16 words mod 64 words the
// four rows one 32-lane pass reads sit on disjoint banks.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ bf16x8 frag_tr(const unsigned char* tile, int ld, int row0, int col0,
                                          int lane) {
  const int g = lane >> 4, r = lane & 15;
  const int row = row0 + 8 * (g >> 1) + (r >> 2);
  const int col = col0 + 16 * (g & 1) + 4 * (r & 3);
  const unsigned char* p = tile + row * ld + col * 2;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 4 * ld));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// ---- direct-to-LDS buffer loads ------------------------------------------------------
constexpr int kBufRsrcWord3 = 0x00020000;   // gfx9 buffer descriptor word 3 (raw, 32-bit data)
typedef int i32x4 __attribute__((ext_vector_type(4)));   // buffer descriptor words
typedef __attribute__((address_space(3))) void lds_ptr_void;

// Buffer descriptor words of [base, base + bytes) (raw buffer, stride 0).
__device__ __forceinline__ i32x4 rsrc_words(const void* base, int bytes) {
  const uint64_t p = (uint64_t)(uintptr_t)base;
  return i32x4{(int)(uint32_t)p, (int)(uint32_t)((p >> 32) & 0xffffu), bytes, kBufRsrcWord3};
}

// 32-bit LDS address of a pointer into a __shared__ array.
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(uintptr_t)(lds_ptr_void*)p;
}

// One direct-to-LDS buffer load (16 bytes per lane into lds + 16 lane; bytes past the
// descriptor's range read as zero), written in asm so that the compiler does not track it:
// the compiler makes the first transposing LDS read after a direct-to-LDS load it knows of
// wait for every such load in flight. Callers order these loads themselves (vmcnt waits
// before the barrier that hands a stage over). The load has no register result; M0
// carries the LDS address.
__device__ __forceinline__ void dma16(i32x4 rsrc, unsigned lds, int voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

// The same for 4 bytes per lane (into lds + 4 lane).
__device__ __forceinline__ void dma4(i32x4 rsrc, unsigned lds, int voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(lds), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

// Wait until at most n (0 .. 15, wave-uniform) of this wave's vector memory operations are
// outstanding.
__device__ __forceinline__ void wait_vmcnt(int n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    case 1: __builtin_amdgcn_s_waitcnt(0x0F71); break;
    case 2: __builtin_amdgcn_s_waitcnt(0x0F72); break;
    case 3: __builtin_amdgcn_s_waitcnt(0x0F73); break;
    case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
    case 5: __builtin_amdgcn_s_waitcnt(0x0F75); break;
    case 6: __builtin_amdgcn_s_waitcnt(0x0F76); break;
    case 7: __builtin_amdgcn_s_waitcnt(0x0F77); break;
    case 8: __builtin_amdgcn_s_waitcnt(0x0F78); break;
    case 9: __builtin_amdgcn_s_waitcnt(0x0F79); break;
    case 10: __builtin_amdgcn_s_waitcnt(0x0F7A); break;
    case 11: __builtin_amdgcn_s_waitcnt(0x0F7B); break;
    case 12: __builtin_amdgcn_s_waitcnt(0x0F7C); break;
    case 13: __builtin_amdgcn_s_waitcnt(0x0F7D); break;
    case 14: __builtin_amdgcn_s_waitcnt(0x0F7E); break;
    default: __builtin_amdgcn_s_waitcnt(0x0F7F); break;
  }
}

// Stage W^T for features [f0, f0+nf) into LDS as [nf][128 d] rows of 256 B, in the K-tile
// layout (row f, chunk c at c ^ kappa(f & 15)). W is [128 d][F] bf16 (row-major).
__device__ __forceinline__ void stage_wt(unsigned char* dst, const uint16_t* W, int F, int f0,
                                         int nf, int tid, int nthreads = 256) {
  // pairs (d, chunk of 8 features): thread reads W[d][f0 + 8c .. +8]
  const int pairs = kDim * (nf / 8);
  for (int id = tid; id < pairs; id += nthreads) {
    int d = id & (kDim - 1), c = id >> 7;
    u32x4 w = *reinterpret_cast<const u32x4*>(W + (int64_t)d * F + f0 + c * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      unsigned x = w[e >> 1];
      uint16_t h = (e & 1) ? (uint16_t)(x >> 16) : (uint16_t)(x & 0xffffu);
      int f = c * 8 + e;
      *reinterpret_cast<uint16_t*>(dst + f * 256 + ((((d >> 3) ^ kappa(f & 15))) << 4) +
                                   ((d & 7) << 1)) = h;
    }
  }
}

}  // namespace rehyat
