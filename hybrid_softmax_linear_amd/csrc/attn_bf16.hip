// attn_bf16.hip - hybrid softmax/linear attention forward on bf16 MFMA (gfx950), D = 128.
//
// One workgroup (8 waves, two per SIMD) computes 256 query rows of one chunk of one head:
//   y = (sum_window exp(q.k/sqrt(D)) v + a^L) / (sum_window exp(q.k/sqrt(D)) + n^L)
// (joint normalisation of the softmax and linear branches, papernotes.org ReHyAt note,
// key design 1; window = the chunk plus To earlier frames, key design 2; linear branch
// a^L = phi(q) S, n^L = phi(q) z from the carried state, key design 4).
//
// Each wave owns 32 queries (one 32-query MFMA column block); the two waves sharing a SIMD
// hide each other's softmax and LDS latency behind their MFMAs. Work is done transposed:
// S^T = K Q^T (A = K from LDS, B = Q^T held in registers), so each lane owns one query
// column and the sums over keys stay inside the lane pair (l, l^32); the exponentiated
// tile P^T feeds O^T = V^T P^T as the B operand without leaving registers. K and V tiles
// ([128 keys][128 d], straight from the q/k/v layout) stream into LDS by buffer loads that
// write LDS directly (no staging registers); rows past the window come back as zeros from
// the buffer descriptor's range check. The V^T operand fragments come from the row-major V
// tile by the transposing LDS read.
//
// The linear branch enters as one extra "key" of weight n^L and value a^L/n^L. All
// exponentials of a query row share one fixed reference m0 (log2 units):
//     m0 = max(log2 n^L, max over the first 32 window keys of q.k*log2(e)/sqrt(D)),
// so O = a^L/n^L * 2^(log2 n^L - m0), l = 2^(log2 n^L - m0) before the key loop, and the
// loop only adds p = 2^(s - m0) terms: O and l are never rescaled inside it (the MFMA
// accumulators are touched by MFMAs only). Every term is an exact power-of-two rescaling
// of the unstabilised weight, so y = O / l is the unstabilised definition. Keys beyond the
// first block may exceed m0; that is harmless while O and l stay finite (fp32 and bf16
// share an 8-bit exponent). If any accumulator of the workgroup ends non-finite, the
// workgroup recomputes with m0 = the exact row maximum over the window (all p <= 1).
#include "partial_bf16.h"

namespace rehyat {

namespace {

constexpr int NW = 8;           // waves per workgroup
constexpr int QW = 32;          // queries per wave
constexpr int NT = NW * 64;     // threads per workgroup
constexpr int QT = NW * QW;     // queries per workgroup
constexpr float kNegBig = -3.0e38f;
constexpr int kKeys = 128;                               // keys per LDS tile
constexpr int kRow = 272;                                // LDS row: 256 B of data + 16 B pad
constexpr int kDmaInsts = kKeys * (kRow / 16) / 64;      // 1 KB DMA instructions per tile (34)
constexpr int kKBytes = kKeys * kRow;                    // K tile [128 keys][128 d] bf16
// V tiles are row-major too, rows padded to 288 B (72 words, 8 mod 64): the transposing
// LDS read that forms the V^T fragments touches 4 rows x 32 bytes per 16 lanes, and that
// stride keeps them on distinct banks.
constexpr int kVRow = 288;                               // V row: 256 B + 32 B pad
constexpr int kVInsts = kKeys * (kVRow / 16) / 64;       // 36
constexpr int kVBytes = kKeys * kVRow;                   // V tile [128 keys][128 d] bf16
constexpr int kStageBytes = kKBytes + kVBytes;           // 70 KB per stage

typedef __attribute__((address_space(3))) void lds_void;

struct QRegs {
  bf16x8 op[8];                 // B operand of S^T = K Q^T: [d step]
};

struct Acc {
  f32x16 O[4];                  // O^T accumulators: [d block]
  float l;                      // partial weight sum of this lane's keys
};

// Per-workgroup geometry of one (head, chunk, query tile).
struct Geo {
  int bh, h, t_local, rows, q_wave0;
  int64_t q_row_base, lo, hi;
  bool has_linear;
};

// Tile sources of one workgroup: K and V rows of the window. The streaming step's window
// is in two segments (the carried tail, then the chunk): window rows [0, na) come from
// k / v, the rest from k2 / v2, whose base sits na rows before the chunk's first row so
// that one byte offset (window row * 256 + column) addresses either segment.
struct Src {
  i32x4 k;                      // base = first window row, range = nk rows (na rows: step)
  i32x4 v;
  i32x4 k2;                     // step: base = chunk row 0 - na rows, range = nk rows
  i32x4 v2;
  int nk;                       // window length
  int na_bytes;                 // step: 256 x the window rows in the first segment
};

__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0)
__device__ __forceinline__ void wait_vmem_lds() { __builtin_amdgcn_s_waitcnt(0x0070); }   // vmcnt(0) lgkmcnt(0)

// Tile layout in LDS: K row r (a key) of 256 B at r * 272, its 16-byte chunk c at + 16 c.
// The 16-byte pad shifts consecutive rows by four banks, so the 16 lanes of a read group
// (16 consecutive rows, one chunk) cover all 64 banks, and every fragment read below is one
// per-lane base plus a constant offset. V row r at r * 288 (see kVRow).

// Descriptor of the rows from byte t0 on: base advanced by t0, range shortened by t0.
__device__ __forceinline__ i32x4 rsrc_from(i32x4 r, int t0) {
  const uint64_t b = ((uint64_t)(uint32_t)r[1] << 32 | (uint32_t)r[0]) + (uint32_t)t0;
  const int left = r[2] - t0;
  return i32x4{(int)(uint32_t)b, (int)(uint32_t)(b >> 32), left > 0 ? left : 0, r[3]};
}

// Issue the direct-to-LDS loads of tile kt into one stage. Each instruction writes 64
// consecutive 16-byte slots (1 KB) of a tile; for K slot u holds row u / 17, chunk u % 17
// (the pad slot, chunk 16, takes a second copy of chunk 0); for V row u / 18, chunk u % 18
// (pad slots 16 and 17 copy chunk 0). 34 + 36 instructions per tile, spread over the 8
// waves. kSplit: a lane whose byte offset lies past na_bytes loads from (k2, v2) instead
// (the two loads of an instruction that straddles the boundary write disjoint lanes' slots).
template <bool kSplit, int kPart = 2>
__device__ __forceinline__ void tile_dma_from(i32x4 k, i32x4 v, const Src& s, int kt,
                                              unsigned char* stage, int wave, int lane) {
  const unsigned sl = lds_addr(stage);
  if (!kSplit) {
    // descriptors that start at the tile: the lanes' offsets are the same for every tile, and
    // the advance is scalar work (rows past the window still read as zeros)
    const int t0 = kt * kKeys * 256;
    if (kPart != 1) k = rsrc_from(k, t0);
    if (kPart != 0) v = rsrc_from(v, t0);
    kt = 0;
  }
#pragma unroll
  for (int i = 0; i < (kPart == 1 ? 0 : (kDmaInsts + NW - 1) / NW); ++i) {
    const int j = wave + NW * i;
    if (j < kDmaInsts) {
      const int u = 64 * j + lane;
      const int r = u / 17;
      int c = u - 17 * r;
      c = c == 16 ? 0 : c;
      const int off = (kt * kKeys + r) * 256 + c * 16;
      if (!kSplit || off < s.na_bytes)
        dma16(k, sl + j * 1024, off);
      else
        dma16(s.k2, sl + j * 1024, off);
    }
  }
#pragma unroll
  for (int i = 0; i < (kPart == 0 ? 0 : (kVInsts + NW - 1) / NW); ++i) {
    const int j = wave + NW * i;
    if (j < kVInsts) {
      const int u = 64 * j + lane;
      const int r = u / 18;
      int c = u - 18 * r;
      c = c >= 16 ? 0 : c;
      const int off = (kt * kKeys + r) * 256 + c * 16;
      if (!kSplit || off < s.na_bytes)
        dma16(v, sl + kKBytes + j * 1024, off);
      else
        dma16(s.v2, sl + kKBytes + j * 1024, off);
    }
  }
}

// kTwo: the window is in two segments. A tile wholly inside one of them takes that
// segment's descriptors (a uniform choice); only the tile that straddles the boundary
// chooses per lane.
// kPart: 0 the K loads, 1 the V loads, 2 both.
template <bool kTwo, int kPart = 2>
__device__ __forceinline__ void tile_dma(const Src& s, int kt, unsigned char* stage, int wave,
                                         int lane) {
  if (!kTwo) {
    tile_dma_from<false, kPart>(s.k, s.v, s, kt, stage, wave, lane);
    return;
  }
  const int t0 = kt * kKeys * 256;
  if (t0 < s.na_bytes && t0 + kKeys * 256 > s.na_bytes) {
    tile_dma_from<true, kPart>(s.k, s.v, s, kt, stage, wave, lane);
  } else if (t0 < s.na_bytes) {
    tile_dma_from<false, kPart>(s.k, s.v, s, kt, stage, wave, lane);
  } else {
    tile_dma_from<false, kPart>(s.k2, s.v2, s, kt, stage, wave, lane);
  }
}

// K fragments (A operand of S^T = K Q^T) of 32-key block kb: lane l takes key row
// 32 kb + kappa(l % 32) (the row order that makes the S^T accumulator the B operand of the
// PV product) at chunks 2 s + l / 32.
__device__ __forceinline__ void load_k(bf16x8 (&kf)[8], const unsigned char* kbuf, int kb,
                                       int lane) {
  const int base = kappa(lane & 31) * kRow + (lane >> 5) * 16;
#pragma unroll
  for (int s = 0; s < 8; ++s) kf[s] = as_bf16x8(lds_read16(kbuf, base + kb * 32 * kRow + s * 32));
}

// V^T fragments (A operand of O^T += V^T P^T) of 32-key block kb: lane l takes column
// d = 32 db + l % 32 of the row-major V tile at keys 32 kb + 16 j + 8 (l / 32) .. + 7, by
// the transposing LDS read.
__device__ __forceinline__ void load_v(bf16x8 (&vf)[4][2], const unsigned char* vbuf, int kb,
                                       int lane) {
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int j = 0; j < 2; ++j)
      vf[db][j] = frag_tr(vbuf, kVRow, 32 * kb + 16 * j, 32 * db, lane);
}

// S^T block (32 keys x 32 queries) from K fragments.
__device__ __forceinline__ f32x16 qk_mfma(const bf16x8 (&kf)[8], const QRegs& Q) {
  f32x16 S;
#pragma unroll
  for (int i = 0; i < 16; ++i) S[i] = 0.0f;
#pragma unroll
  for (int s = 0; s < 8; ++s) S = mfma32(kf[s], Q.op[s], S);
  return S;
}

// S^T block of 32-key block kb, all eight K fragments in flight before the first MFMA.
__device__ __forceinline__ f32x16 qk_block(const unsigned char* kbuf, int kb, const QRegs& Q,
                                           int lane) {
  bf16x8 kf[8];
  load_k(kf, kbuf, kb, lane);
  f32x16 S = qk_mfma(kf, Q);
  __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
  return S;
}

__device__ __forceinline__ void mask_block(f32x16& S, int key0, int nk, int lane) {
#pragma unroll
  for (int i = 0; i < 16; ++i)
    if (key0 + cidx(i, lane) >= nk) S[i] = -__builtin_inff();
}

__device__ __forceinline__ float rowmax16(const f32x16& v) {
  float m = fmaxf(fmaxf(v[0], v[1]), v[2]);
#pragma unroll
  for (int i = 3; i < 15; i += 2) m = fmaxf(fmaxf(m, v[i]), v[i + 1]);
  return fmaxf(m, v[15]);
}

// p = 2^(s*ls - m0) as bf16 (the B operand of O^T += V^T P^T); l += sum of the rounded p.
__device__ __forceinline__ void softmax_block(bf16x8 (&P)[2], float& l, const f32x16& S,
                                              float m0, float ls) {
  const bf16x2 ones{(bf16)1.0f, (bf16)1.0f};
  float acc = 0.0f;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    u32x4 pk;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i0 = 8 * j + 2 * e;
      bf16x2 pb = pack_bf16(fast_exp2(S[i0] * ls - m0), fast_exp2(S[i0 + 1] * ls - m0));
      acc = __builtin_amdgcn_fdot2_f32_bf16(pb, ones, acc, false);
      pk[e] = __builtin_bit_cast(unsigned, pb);
    }
    P[j] = as_bf16x8(pk);
  }
  l += acc;
}

__device__ __forceinline__ void pv_mfma(Acc& A, const bf16x8 (&vf)[4][2], const bf16x8 (&P)[2]) {
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int db = 0; db < 4; ++db) A.O[db] = mfma32(vf[db][j], P[j], A.O[db]);
}

// Raw-operand staging (streaming step, where S is the caller's fp32 state): W slab
// [128 d][FS] row-major at kWRow-byte rows, the 4-feature blocks of each 16 in the order
// kappa (positions 4..7 and 8..11 swapped), so that the transposing read of physical
// column 32 fb + (l mod 32) hands lane l the W^T row 32 fb + kappa(l mod 32) of the image
// layout; bytes of the W slab, then the S^T slab.
constexpr int kWRow = 288;
constexpr int kWRawBytes = kDim * kWRow;

// W[d][f0 .. f0+FS) of a [128][F] bf16 W into the raw W slab.
template <int F, int FS>
__device__ __forceinline__ void stage_w_raw(unsigned char* wt, const uint16_t* W, int f0, int tid) {
#pragma unroll
  for (int it = 0; it < (kDim * FS / 8 + NT - 1) / NT; ++it) {
    const int id = it * NT + tid;
    if (id < kDim * FS / 8) {
      const int d = id / (FS / 8), c = id % (FS / 8);
      const u32x4 w = *reinterpret_cast<const u32x4*>(W + (int64_t)d * F + f0 + 8 * c);
      const int col = 16 * (c >> 1) + ((c & 1) ? 4 : 0);   // logical block 2(c&1) -> kappa
      unsigned char* row = wt + d * kWRow;
      *reinterpret_cast<uint2*>(row + col * 2) = uint2{w[0], w[1]};
      *reinterpret_cast<uint2*>(row + (col + 8) * 2) = uint2{w[2], w[3]};
    }
  }
}

// S[f0 .. f0+FS)[0 .. 128) (fp32) into the S^T slab: rows d of FS bf16, feature chunk c at
// chunk c ^ (d mod FS/8), the layout (and rounding) of the S^T image.
template <int FS>
__device__ __forceinline__ void stage_st_raw(unsigned char* st, const float* S, int f0, int tid) {
  constexpr int NCH = FS / 8;
#pragma unroll
  for (int it = 0; it < (kDim * NCH + NT - 1) / NT; ++it) {
    const int id = it * NT + tid;
    if (id < kDim * NCH) {
      const int d = id & (kDim - 1), c = id >> 7;
      const float* src = S + (int64_t)(f0 + 8 * c) * kDim + d;
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = pack_bf16_u32(src[(2 * e) * kDim], src[(2 * e + 1) * kDim]);
      *reinterpret_cast<u32x4*>(st + d * (FS * 2) + ((c ^ (d & (NCH - 1))) << 4)) = w;
    }
  }
}

// Linear branch: O = a^L^T = S^T phi(Q)^T (bf16 MFMA) and n^L = phi(q).z (full sum over
// the lane pair). The W^T and S^T slabs of FS features come from bf16 images already in
// the LDS layout (W^T rows f at chunk c ^ kappa(f & 15); S^T rows d at chunk
// c ^ (d mod FS/8)) and are copied into `stage` (64 KB) by direct-to-LDS loads; with kRaw
// they are staged from W and the fp32 state through registers (same operand values, so
// the same bits). Ends with a barrier.
template <int F, bool kRaw>
__device__ __forceinline__ void linear_branch(Acc& A, float& nlf, const AttnArgs& a,
                                              const Geo& g, const QRegs& Q, unsigned char* stage,
                                              float* zs, int tid, int lane, const uint16_t* pqrow) {
  const int wave = tid >> 6;
  const float* z = a.z + g.bh * a.z_bh + g.t_local * a.z_t;
  float nl = 0.0f;
  for (int f = tid; f < F; f += NT) zs[f] = z[f];
  constexpr int FS = F < 128 ? F : 128;   // features per LDS slab
  constexpr int NFB = FS / 32;            // 32-feature blocks per slab
  const float c1 = a.u_scale, c2 = 0.5f * a.u_scale * a.u_scale;
  constexpr int NCH = FS / 8;             // 16-byte chunks per S^T row
  constexpr int SLAB = FS * 256;          // bytes of one W^T slab and of one S^T slab
  const unsigned char* wimg = reinterpret_cast<const unsigned char*>(a.wt_img) +
                              (a.w_per_head ? (int64_t)g.h * a.wt_img_head : 0);
  const unsigned char* simg = reinterpret_cast<const unsigned char*>(a.st_img) +
                              g.bh * a.st_img_bh + g.t_local * a.st_img_t;
  const __amdgpu_buffer_rsrc_t wr =
      __builtin_amdgcn_make_buffer_rsrc((void*)wimg, (short)0, F * 256, kBufRsrcWord3);
  const __amdgpu_buffer_rsrc_t sr =
      __builtin_amdgcn_make_buffer_rsrc((void*)simg, (short)0, F * 256, kBufRsrcWord3);
  unsigned char* wt = stage;                               // [FS][128] bf16 (raw: [128][FS])
  unsigned char* st = stage + (kRaw ? kWRawBytes : 32768);  // [128 d][FS] bf16
  const uint16_t* wraw = reinterpret_cast<const uint16_t*>(a.Wq) +
                         (a.w_per_head ? (int64_t)g.h * kDim * F : 0);
  const float* sraw = a.S + g.bh * a.s_bh + g.t_local * a.s_t;
#pragma unroll 1
  for (int f0 = 0; f0 < F; f0 += FS) {
    if (f0 > 0) __syncthreads();
    if (kRaw) {
      if (!a.phiq) stage_w_raw<F, FS>(wt, wraw, f0, tid);
      stage_st_raw<FS>(st, sraw, f0, tid);
    } else {
      const int base = (f0 / FS) * SLAB;
#pragma unroll
      for (int i = 0; i < (SLAB / 1024 + NW - 1) / NW; ++i) {
        const int j = wave + NW * i;
        if (j < SLAB / 1024) {
          if (!a.phiq)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_void*)(wt + j * 1024), 16,
                                                     base + j * 1024 + lane * 16, 0, 0, 0);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(sr, (lds_void*)(st + j * 1024), 16,
                                                   base + j * 1024 + lane * 16, 0, 0, 0);
        }
      }
      wait_vmem();
    }
    __syncthreads();
    // U^T blocks: rows = features 32fb + kappa(l%32) (A = W^T), cols = queries (B = Q^T);
    // G chains at a time (fewer for F = 256, whose slab loop keeps more state live).
    constexpr int G = F > 128 ? 2 : NFB;
#pragma unroll
    for (int fg = 0; fg < NFB; fg += G) {
      bf16x8 P[G][2];
      if (a.phiq) {
        // phi(q) computed ahead: this lane's 8 consecutive features per operand
#pragma unroll
        for (int k = 0; k < G; ++k)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int fbase = f0 + 32 * (fg + k) + 16 * j + 8 * (lane >> 5);
            const u32x4 w4 = pqrow ? *reinterpret_cast<const u32x4*>(pqrow + fbase)
                                   : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int e = 0; e < 4; ++e)
              nl += bf16_lo(w4[e]) * zs[fbase + 2 * e] + bf16_hi(w4[e]) * zs[fbase + 2 * e + 1];
            P[k][j] = as_bf16x8(w4);
          }
      } else {
      f32x16 U[G];
#pragma unroll
      for (int k = 0; k < G; ++k)
#pragma unroll
        for (int i = 0; i < 16; ++i) U[k][i] = 0.0f;
#pragma unroll
      for (int s = 0; s < 8; ++s)
#pragma unroll
        for (int k = 0; k < G; ++k) {
          bf16x8 av;
          if (kRaw) {
            av = frag_tr(wt, kWRow, 16 * s, 32 * (fg + k), lane);
          } else {
            const int arow = 32 * (fg + k) + kappa(lane & 31);
            av = as_bf16x8(lds_read16(wt, ktile_off(arow, 2 * s + (lane >> 5))));
          }
          U[k] = mfma32(av, Q.op[s], U[k]);
        }
      // phi = 1 + u + u^2/2 with u = U / sqrt(D), as 1 + U (c1 + c2 U) (c1 = 1/sqrt(D),
      // c2 = c1^2 / 2), rounded to bf16: B operand of a^L^T = S^T phi^T; n^L takes phi in fp32
#pragma unroll
      for (int k = 0; k < G; ++k)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          u32x4 pk;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i0 = 8 * j + 2 * e;
            const float p0 = fmaf(U[k][i0], fmaf(U[k][i0], c2, c1), 1.0f);
            const float p1 = fmaf(U[k][i0 + 1], fmaf(U[k][i0 + 1], c2, c1), 1.0f);
            pk[e] = pack_bf16_u32(p0, p1);
            const int f = f0 + 32 * (fg + k) + cidx(i0, lane);
            nl = fmaf(p0, zs[f], nl);
            nl = fmaf(p1, zs[f + 1], nl);
          }
          P[k][j] = as_bf16x8(pk);
        }
      }
#pragma unroll
      for (int k = 0; k < G; ++k)
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const int d = 32 * db + (lane & 31);
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int c = 4 * (fg + k) + 2 * j + (lane >> 5);
            bf16x8 av = as_bf16x8(lds_read16(st, d * (FS * 2) + ((c ^ (d & (NCH - 1))) << 4)));
            A.O[db] = mfma32(av, P[k][j], A.O[db]);
          }
        }
    }
  }
  nlf = pair_sum(nl);
  __syncthreads();
}

__device__ __forceinline__ void zero_acc(Acc& A) {
  A.l = 0.0f;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) A.O[db][i] = 0.0f;
}

// With O = a^L (from linear_branch) and reference m0: O = a^L/n^L * w, l = w (in one lane
// of the pair), w = n^L 2^(-m0) computed as sign(n^L) 2^(log2 |n^L| - m0), the weight of the
// linear "key". (Learned feature maps can make n^L zero or negative: the scale then stays
// 2^(-m0) and the sign is kept; for n^L > 0 this is exactly w = 2^(log2 n^L - m0).)
__device__ __forceinline__ void scale_linear(Acc& A, float nl, float m0, int lane) {
  const float an = fabsf(nl);
  const float w = fast_exp2(fast_log2(an) - m0);
  const float sc = an > 0.0f ? w / an : fast_exp2(-m0);
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) A.O[db][i] *= sc;
  A.l = (lane < 32) ? __builtin_copysignf(w, nl) : 0.0f;
}

// One 128-key tile from LDS: four 32-key blocks of S^T = K Q^T, p = 2^(s*ls - m0),
// l += sum p, O^T += V^T P^T. The last tile of the window masks keys >= nk.
// LDS reads run one block ahead of the MFMAs that use them: kf and vf hold block 0's K and
// V^T fragments on entry, and each block requests the next block's fragments right after
// its S^T MFMAs, so they arrive while the exponentials and PV MFMAs run. In a tile that is
// not the window's last, the barrier that hands over the next stage sits inside block 3:
// once this wave's reads of the current stage have returned and its share of the next
// tile has landed, the barrier passes and the next tile's block-0 fragments are requested
// before block 3's exponentials (kf and vf hold them on exit), so the pipeline does not
// drain at tile boundaries.
template <bool kLastTile, bool kTwo>
__device__ __forceinline__ void process_tile(Acc& A, float m0, const unsigned char* stage,
                                             unsigned char* next_stage, int kt, int nk,
                                             const QRegs& Q, float ls, int wave, int lane,
                                             const Src& src, bf16x8 (&kf)[8],
                                             bf16x8 (&vf)[4][2]) {
  const unsigned char* kbuf = stage;
  const unsigned char* vbuf = stage + kKBytes;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const int key0 = kt * kKeys + kb * 32;
    if (kLastTile && key0 >= nk) break;
    f32x16 S = qk_mfma(kf, Q);
    // the next tile's loads, in two parts under the first two blocks' MFMAs (the stage they
    // fill was released at the last tile's barrier)
    if (!kLastTile && kb == 0) tile_dma<kTwo, 0>(src, kt + 1, next_stage, wave, lane);
    if (!kLastTile && kb == 1) tile_dma<kTwo, 1>(src, kt + 1, next_stage, wave, lane);
    bf16x8 vn[4][2];
    if (kb < 3) {
      load_k(kf, kbuf, kb + 1, lane);
      load_v(vn, vbuf, kb + 1, lane);
    } else if (!kLastTile) {
      wait_vmem_lds();
      __syncthreads();
      load_k(kf, next_stage, 0, lane);
      load_v(vn, next_stage + kKBytes, 0, lane);
    }
    if (kLastTile) mask_block(S, key0, nk, lane);
    bf16x8 P[2];
    softmax_block(P, A.l, S, m0, ls);
    pv_mfma(A, vf, P);
    if (kb < 3 || !kLastTile) {
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        vf[db][0] = vn[db][0];
        vf[db][1] = vn[db][1];
      }
    }
  }
}

// Exact row maximum over the window (log2 units), for the overflow fallback.
template <bool kTwo>
__device__ __forceinline__ float max_sweep(const Src& src, const QRegs& Q, unsigned char* smem,
                                           float ls, int wave, int lane) {
  const int ntiles = (src.nk + kKeys - 1) / kKeys;
  float mx = kNegBig;
#pragma unroll 1
  for (int kt = 0; kt < ntiles; ++kt) {
    __syncthreads();
    tile_dma<kTwo>(src, kt, smem, wave, lane);
    wait_vmem();
    __syncthreads();
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      f32x16 S = qk_block(smem, kb, Q, lane);
      mask_block(S, kt * kKeys + kb * 32, src.nk, lane);
      mx = fmaxf(mx, rowmax16(S) * ls);
    }
  }
  mx = pair_max(mx);
  __syncthreads();
  return mx;
}

// The key loop over a window whose tile 0 is already in stage 0: double-buffered
// direct-to-LDS tiles, one barrier per tile, the last tile peeled (masking).
// Waves without a query tile (in workgroups that hold 7 of the chunk's wave tiles) only
// help with the tile loads and barriers.
template <bool kTwo>
__device__ __forceinline__ void key_loop(Acc& A, float m0, const Src& src, const QRegs& Q,
                                         unsigned char* smem, float ls, int wave, int lane,
                                         bool active) {
  const int nk = src.nk;
  const int ntiles = (nk + kKeys - 1) / kKeys;
  bf16x8 kf[8], vf[4][2];
  if (active) {
    load_k(kf, smem, 0, lane);
    load_v(vf, smem + kKBytes, 0, lane);
  }
#pragma unroll 1
  for (int kt = 0; kt < ntiles - 1; ++kt) {
    unsigned char* cur = smem + (kt & 1) * kStageBytes;
    unsigned char* nxt = smem + ((kt & 1) ^ 1) * kStageBytes;
    if (active) {
      process_tile<false, kTwo>(A, m0, cur, nxt, kt, nk, Q, ls, wave, lane, src, kf, vf);
    } else {
      tile_dma<kTwo>(src, kt + 1, nxt, wave, lane);
      wait_vmem_lds();
      __syncthreads();
    }
  }
  const int kt = ntiles - 1;
  if (active)
    process_tile<true, kTwo>(A, m0, smem + (kt & 1) * kStageBytes, smem, kt, nk, Q, ls, wave, lane,
                             src, kf, vf);
  __syncthreads();
}

// Wait for window tile 0 in stage 0 (its loads were issued by the caller) and fix the
// reference: max(mlow, block-0 row maximum).
__device__ __forceinline__ float start_window(float mlow, const Src& src, const QRegs& Q,
                                              unsigned char* smem, float ls, int wave, int lane) {
  wait_vmem();
  __syncthreads();
  f32x16 S = qk_block(smem, 0, Q, lane);
  if (src.nk < 32) mask_block(S, 0, src.nk, lane);
  return fmaxf(mlow, pair_max(rowmax16(S)) * ls);
}

// Work order. Blocks are handed to the XCDs round-robin (block b to XCD b mod 8) and each
// XCD starts its blocks in order as CUs free up. Each XCD first takes its share of the
// tiles of chunks 1 .. n_chunks-1, then its share of chunk 0's tiles, whose window lacks the
// overlap frames: the last workgroups to start are the short ones. Within a share an XCD
// takes consecutive tiles of one window, which then share its L2. Returns (head, chunk
// within the launch, query tile) of block b.
__device__ __forceinline__ void tile_of_block(const AttnArgs& a, int b, int& bh, int& t_local,
                                              int& qt) {
  const int nb = a.nblocks, nch = a.n_chunks;
  const int tpc = a.tiles_per_chunk, tl = a.tiles_last;
  const int BH = nb / a.tiles_per_head;
  const int ntile0 = nch == 1 ? tl : tpc;
  const int H = nb - BH * ntile0;                   // tiles of chunks 1 .. nch-1
  const int x = b & 7, i = b >> 3;
  const int hq = H >> 3, hr = H & 7;
  const int hcnt = hq + (x < hr ? 1 : 0);
  const int hstart = x * hq + (x < hr ? x : hr);
  int item;
  if (i < hcnt) {
    item = hstart + i;
  } else {
    const int before = x * (nb >> 3) + (x < (nb & 7) ? x : (nb & 7));   // blocks of XCDs < x
    item = H + (before - hstart) + (i - hcnt);
  }
  if (item < H) {
    const int mid = (nch - 2) * BH * tpc;           // tiles of chunks 1 .. nch-2
    if (item < mid) {
      const int c = item / (BH * tpc), r = item - c * BH * tpc;
      t_local = c + 1;
      bh = r / tpc;
      qt = r - bh * tpc;
    } else {
      const int r = item - mid;
      t_local = nch - 1;
      bh = r / tl;
      qt = r - bh * tl;
    }
  } else {
    const int r = item - H;
    t_local = 0;
    bh = r / ntile0;
    qt = r - bh * ntile0;
  }
}

// One attention workgroup: query tile `b` of the launch (in tile_of_block's order). smem:
// 140 KB, two K/V stages during the key loop, W^T and S^T slabs for the linear branch.
// kTwo: the window in two segments (the streaming step's carried tail, then the chunk);
// kRaw: the linear operands staged from W and the fp32 state. Returns the head.
template <int F, bool kTwo, bool kRaw>
__device__ __forceinline__ int attention_block(const AttnArgs& a, int b, unsigned char* smem,
                                               float* zs, int& bad_flag) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  Geo g;
  int qt;
  tile_of_block(a, b, g.bh, g.t_local, qt);
  const int t = a.chunk0 + g.t_local;
  g.h = g.bh % a.H;
  const int64_t Np = (int64_t)a.Tc * a.HW;
  const int64_t N = (int64_t)a.T * a.HW;
  const int64_t c0 = t * Np;                                  // first token of the chunk
  g.rows = (int)((N - c0) < Np ? (N - c0) : Np);               // query rows of the chunk
  g.lo = (c0 - (int64_t)a.To * a.HW) > 0 ? (c0 - (int64_t)a.To * a.HW) : 0;
  g.hi = c0 + g.rows;
  g.has_linear = a.bidir ? (g.lo > 0 || g.hi < N) : (g.lo > 0);
  // The chunk's 32-query wave tiles are split evenly over its workgroups (7 or 8 per
  // workgroup), so no workgroup holds a mostly idle last tile.
  const int ntile_c = (g.t_local == a.n_chunks - 1) ? a.tiles_last : a.tiles_per_chunk;
  const int nwt = (g.rows + QW - 1) / QW;
  const int wt0 = (qt * nwt) / ntile_c, wt1 = ((qt + 1) * nwt) / ntile_c;
  const bool active = wt0 + wave < wt1;   // wave-uniform
  g.q_wave0 = (wt0 + wave) * QW;
  g.q_row_base = a.step ? 0 : c0;   // row of the chunk start in the q buffer
  if (tid == 0) bad_flag = 0;

  // ---- Q^T operand registers ----------------------------------------------------------
  const uint16_t* qh = reinterpret_cast<const uint16_t*>(a.q) + head_off(g.bh, a.q_rows, kDim);
  const int qrow = g.q_wave0 + (lane & 31);
  QRegs Q;
  {
    const bool ok = active && qrow < g.rows;
    const uint16_t* src = qh + (g.q_row_base + (ok ? qrow : 0)) * kDim + 8 * (lane >> 5);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      u32x4 v = ok ? *reinterpret_cast<const u32x4*>(src + 16 * s) : u32x4{0u, 0u, 0u, 0u};
      Q.op[s] = as_bf16x8(v);
    }
  }

  // ---- tile sources: K and V rows of the window ---------------------------
  Src src;
  {
    const int nk = (int)(g.hi - g.lo);
    src.nk = nk;
    if (kTwo) {
      // rows [0, na): the last na rows of the tail (segment A); then the chunk (segment B),
      // addressed from na rows before its start (no access below the chunk: a lane takes
      // segment B only for offsets >= na * 256)
      const int na = (int)(c0 - g.lo);
      src.na_bytes = na * 256;
      const int64_t ah = head_off(g.bh, a.a_rows, kDim) + (a.a_rows - na) * kDim;
      const int64_t bh0 = head_off(g.bh, a.b_rows, kDim) - (int64_t)na * kDim;
      src.k = rsrc_words(reinterpret_cast<const uint16_t*>(a.ka) + ah, na * 256);
      src.v = rsrc_words(reinterpret_cast<const uint16_t*>(a.va) + ah, na * 256);
      src.k2 = rsrc_words(reinterpret_cast<const uint16_t*>(a.kb) + bh0, nk * 256);
      src.v2 = rsrc_words(reinterpret_cast<const uint16_t*>(a.vb) + bh0, nk * 256);
    } else {
      src.na_bytes = nk * 256;
      const uint16_t* kbase = reinterpret_cast<const uint16_t*>(a.ka) +
                              head_off(g.bh, a.a_rows, kDim) + (a.step ? 0 : g.lo) * kDim;
      src.k = rsrc_words(kbase, nk * 256);
      const uint16_t* vbase = reinterpret_cast<const uint16_t*>(a.va) +
                              head_off(g.bh, a.a_rows, kDim) + (a.step ? 0 : g.lo) * kDim;
      src.v = rsrc_words(vbase, nk * 256);
      src.k2 = src.k;
      src.v2 = src.v;
    }
  }
  const float ls = a.logit_scale;

  // ---- linear branch, reference m0, key loop ------------------------------------------
  // Window tile 0 streams into stage 0 while the linear branch stages its operands in
  // stage 1.
  tile_dma<kTwo>(src, 0, smem, wave, lane);
  Acc A;
  float nl = 1.0f, ml = kNegBig;
  zero_acc(A);
  const uint16_t* pqrow =
      (a.phiq && active && qrow < g.rows)
          ? reinterpret_cast<const uint16_t*>(a.phiq) +
                ((int64_t)g.bh * a.q_rows + g.q_row_base + qrow) * F
          : nullptr;
  if (g.has_linear) {
    linear_branch<F, kRaw>(A, nl, a, g, Q, smem + kStageBytes, zs, tid, lane, pqrow);
    ml = fast_log2(fabsf(nl));
  }
  float m0 = start_window(ml, src, Q, smem, ls, wave, lane);
  if (g.has_linear) scale_linear(A, nl, m0, lane);
  key_loop<kTwo>(A, m0, src, Q, smem, ls, wave, lane, active);

  // ---- overflow guard: recompute the workgroup with the exact row maxima ---------------
  {
    bool bad = !__builtin_isfinite(A.l);
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) bad |= !__builtin_isfinite(A.O[db][i]);
    if (wave_any(bad) && lane == 0) atomicOr(&bad_flag, 1);
    __syncthreads();
    if (bad_flag) {
      const float mx = max_sweep<kTwo>(src, Q, smem, ls, wave, lane);
      zero_acc(A);
      tile_dma<kTwo>(src, 0, smem, wave, lane);
      if (g.has_linear)
        linear_branch<F, kRaw>(A, nl, a, g, Q, smem + kStageBytes, zs, tid, lane, pqrow);
      // reference = the exact maximum over the linear weight and every window key: every
      // p <= 1 and l >= 1
      m0 = start_window(fmaxf(ml, mx), src, Q, smem, ls, wave, lane);
      if (g.has_linear) scale_linear(A, nl, m0, lane);
      key_loop<kTwo>(A, m0, src, Q, smem, ls, wave, lane, active);
    }
  }

  // ---- epilogue: y = O / l ------------------------------------------------------------
  const float ltot = pair_sum(A.l);
  const float inv = 1.0f / ltot;
  if (a.lse && active && qrow < g.rows && lane < 32)
    a.lse[(int64_t)g.bh * a.q_rows + g.q_row_base + qrow] = m0 + fast_log2(ltot);
  if (active && qrow < g.rows) {
    const int64_t off = head_off(g.bh, a.q_rows, kDim) + (g.q_row_base + qrow) * kDim;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        const int d = 32 * db + 8 * gi + 4 * (lane >> 5);
        float v0 = A.O[db][4 * gi + 0] * inv, v1 = A.O[db][4 * gi + 1] * inv;
        float v2 = A.O[db][4 * gi + 2] * inv, v3 = A.O[db][4 * gi + 3] * inv;
        if (a.y_f32) {
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.y) + off + d) = f32x4{v0, v1, v2, v3};
        } else {
          uint2 w;
          w.x = pack_bf16_u32(v0, v1);
          w.y = pack_bf16_u32(v2, v3);
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.y) + off + d) = w;
        }
      }
    }
  }
  return g.bh;
}

// The next query tile for a persistent workgroup on XCD home: block indices b = x + 8 j of
// queue x are the blocks the hardware would have placed on XCD x (tile_of_block keeps a
// window's tiles on one XCD), taken in order from the home queue, then from the others
// once it is empty. -1: no work left.
__device__ __forceinline__ int next_tile(unsigned* queue, int nblocks, int home) {
  for (int k = 0; k < kAttnQueues; ++k) {
    const int x = (home + k) & (kAttnQueues - 1);
    const unsigned j = atomicAdd(queue + x, 1u);
    const int64_t b = x + (int64_t)kAttnQueues * j;
    if (b < nblocks) return (int)b;
  }
  return -1;
}

__device__ __forceinline__ int xcd_id() {
  unsigned v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return (int)(v & (kAttnQueues - 1));
}

// One query tile per workgroup, or (kPersistent, a.queue set) one workgroup per compute
// unit taking tiles from per-XCD queues until none is left: the tail of the launch then
// balances over every XCD instead of ending with the XCD that drew the most work. Two
// kernels, so that the loop's registers do not weigh on the one-tile form.
template <int F, bool kPersistent>
__global__ void __launch_bounds__(NT)
__attribute__((amdgpu_waves_per_eu(2, 2)))
hybrid_attn_bf16_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * kStageBytes];
  __shared__ float zs[F];
  __shared__ int bad_flag;
  if (!kPersistent) {
    attention_block<F, false, false>(a, blockIdx.x, smem, zs, bad_flag);
    return;
  }
  __shared__ int tile_s;
  const int home = xcd_id();
  for (;;) {
    if (threadIdx.x == 0) tile_s = next_tile(a.queue, a.nblocks, home);
    __syncthreads();
    const int b = tile_s;
    __syncthreads();   // every thread holds b before thread 0 may take the next tile
    if (b < 0) break;
    attention_block<F, false, false>(a, b, smem, zs, bad_flag);
  }
}

// ---- single-launch recurrent step ------------------------------------------------------
// One launch does the whole step of the chunk-wise RNN (papernotes.org ReHyAt note, key
// design 4): the attention workgroups of the chunk (window = carried tail + chunk, linear
// branch from the carried S, z), one fold workgroup per head and, in the last workgroup of
// each head to finish, the update of S and z.
//   * The fold workgroup forms the per-frame partial sums of the window rows that no later
//     window reaches, two frames at a time (one per half of the workgroup; at F = 256 one
//     frame split over the halves) with the state kernel's operand values and MFMA order,
//     and adds them onto S, z in frame order, exactly as the fold kernel does, into a
//     workspace copy xs. The chunk's last To frames go to the new tail, a buffer apart from
//     the carried one: copied by the grid's padding workgroups (the fold workgroups are
//     padded to a multiple of 8), or by the fold workgroups when there are none.
//   * Every workgroup of a head reports to the head's counter (an agent-scope atomic add)
//     once its reads of S, z and the carried tail have returned; the one that completes the
//     count is the only one left that could read S and z, and copies xs into them.
// No workgroup waits for another. The only data that crosses workgroups inside the launch
// is xs, and it is ordered by a release/acquire pair at agent scope: the fold workgroup's
// add is a release (after the workgroup barrier that follows its xs stores), the other
// workgroups' relaxed adds continue its release sequence, and the last workgroup issues an
// acquire fence after its add and before it reads xs. Only the fold workgroup and the last
// workgroup of a head pay for the cache write-back and invalidate these imply; a release
// in every workgroup cost more than the whole fold. The reads of S and z need no fence:
// each workgroup consumes their values before the barrier ahead of its add, and the last
// workgroup stores only after its add has returned the final count.

// The new tail of head bh: the chunk's last trow rows of K and V (16-byte units, four per
// tensor in flight per thread).
__device__ __forceinline__ void copy_tail(const StepArgs& s, int bh, int tid) {
  const int64_t units = s.trow * (kDim * 2 / 16);
  const u32x4* kc = reinterpret_cast<const u32x4*>(s.kc) +
                    ((int64_t)bh * s.crow + (s.crow - s.trow)) * (kDim * 2 / 16);
  const u32x4* vc = reinterpret_cast<const u32x4*>(s.vc) +
                    ((int64_t)bh * s.crow + (s.crow - s.trow)) * (kDim * 2 / 16);
  u32x4* kt = reinterpret_cast<u32x4*>(s.ktail) + (int64_t)bh * units;
  u32x4* vt = reinterpret_cast<u32x4*>(s.vtail) + (int64_t)bh * units;
#pragma unroll 1
  for (int64_t u0 = tid; u0 < units; u0 += 4 * NT) {
    u32x4 kx[4], vx[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t u = u0 + (int64_t)j * NT;
      if (u < units) {
        kx[j] = kc[u];
        vx[j] = vc[u];
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t u = u0 + (int64_t)j * NT;
      if (u < units) {
        kt[u] = kx[j];
        vt[u] = vx[j];
      }
    }
  }
}

// The fold workgroup of head bh: xs = ((S + p_0) + p_1) + ... over the nseg frames (S taken
// as 0 for the first chunk), then (copy) the new tail. Each round the two halves of the workgroup
// form two frames' partials (F <= 128) or the two halves of one frame's (F = 256, whose
// two feature blocks per wave would not fit beside the attention code's registers) and
// store them (pp: [2][F*D + F]); then all threads add them on elementwise, in frame order.
template <int F>
__device__ __forceinline__ void fold_head(const StepArgs& s, int bh, unsigned char* smem, int tid,
                                          bool copy) {
  constexpr int E = F * kDim + F;
  constexpr bool kSplit = F > 128;
  constexpr int kPer = kSplit ? 1 : 2;   // frames per round
  const int nseg = s.fold.n_seg;
  const int half = tid >> 8, htid = tid & 255;
  float* xs = s.xs + (int64_t)bh * E;
  float* pp = s.pp + (int64_t)bh * 2 * E;
  const float* S0 = s.S + (int64_t)bh * F * kDim;
  const float* z0 = s.z + (int64_t)bh * F;
  if (nseg > 0) {
    const uint16_t* W = reinterpret_cast<const uint16_t*>(s.fold.Wk) +
                        (s.fold.w_per_head ? (int64_t)(bh % s.fold.H) * kDim * F : 0);
    stage_wt(smem, W, F, 0, F, tid, NT);
  }
  unsigned char* tiles = smem + F * 256 + half * kPartialTileBytes;
#pragma unroll 1
  for (int r = 0; kPer * r < nseg; ++r) {
    if (kSplit) {
      const int seg = r;
      const int ntiles = segment_tiles(s.fold, seg);
      if (half == 0) {
        PartialRegs<F, 0> R;
        segment_sums<F, 0>(R, s.fold, bh, seg, ntiles, smem, tiles, tiles + kKTileBytes, htid);
        if (partial_active<F, 0>(seg, htid))
          for_partial<F, 0>(R, htid, [&](int e, float v) { pp[e] = v; });
      } else {
        PartialRegs<F, 1> R;
        segment_sums<F, 1>(R, s.fold, bh, seg, ntiles, smem, tiles, tiles + kKTileBytes, htid);
        if (partial_active<F, 1>(seg, htid))
          for_partial<F, 1>(R, htid, [&](int e, float v) { pp[e] = v; });
      }
    } else {
      const int seg = (2 * r + half < nseg) ? 2 * r + half : -1;
      PartialRegs<F> R;
      segment_sums<F>(R, s.fold, bh, seg, segment_tiles(s.fold, 2 * r), smem, tiles,
                      tiles + kKTileBytes, htid);
      if (partial_active<F>(seg, htid)) {
        float* out = pp + half * E;
        for_partial<F>(R, htid, [&](int e, float v) { out[e] = v; });
      }
    }
    __syncthreads();   // the round's partials stored (workgroup scope)
    const bool pair = !kSplit && 2 * r + 1 < nseg;
#pragma unroll 1
    for (int e = 4 * tid; e < E; e += 4 * NT) {
      f32x4 x;
      if (r > 0)
        x = *reinterpret_cast<const f32x4*>(xs + e);
      else if (s.init)
        x = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      else
        x = *reinterpret_cast<const f32x4*>(e < F * kDim ? S0 + e : z0 + (e - F * kDim));
      x += *reinterpret_cast<const f32x4*>(pp + e);
      if (pair) x += *reinterpret_cast<const f32x4*>(pp + E + e);
      *reinterpret_cast<f32x4*>(xs + e) = x;
    }
    __syncthreads();   // pp free for the next round
  }
  // the new tail, unless the grid's padding workgroups copy it
  if (copy) copy_tail(s, bh, tid);
}


// The last workgroup of head bh: S, z <- xs (or 0 for a first chunk with nothing folded).
template <int F>
__device__ __forceinline__ void finish_head(const StepArgs& s, int bh, int tid) {
  constexpr int E = F * kDim + F;
  float* Sd = s.S + (int64_t)bh * F * kDim;
  float* zd = s.z + (int64_t)bh * F;
  const float* xs = s.xs + (int64_t)bh * E;
  const bool copy = s.fold.n_seg > 0;
  for (int e = 4 * tid; e < E; e += 4 * NT) {
    float* dst = e < F * kDim ? Sd + e : zd + (e - F * kDim);
    f32x4 x = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    if (copy) x = *reinterpret_cast<const f32x4*>(xs + e);
    if (copy || s.init) *reinterpret_cast<f32x4*>(dst) = x;
  }
}

template <int F>
__global__ void __launch_bounds__(NT)
__attribute__((amdgpu_waves_per_eu(2, 2)))
recurrent_step_bf16_kernel(AttnArgs a, StepArgs s) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * kStageBytes];
  __shared__ float zs[F];
  __shared__ int bad_flag;
  __shared__ int last_flag;
  static_assert(F * 256 + 2 * kPartialTileBytes <= 2 * kStageBytes, "fold tiles exceed LDS");
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int BH = a.nblocks / a.tiles_per_head;
  int bh;
  if (b < s.fold_blocks) {
    if (b >= BH) {
      // padding workgroup (the fold workgroups are padded to a multiple of 8): copies the new
      // tails of heads b - BH, b - BH + P, ... (P padding workgroups), which takes the copy
      // off the fold workgroups; reports nowhere
      for (int h = b - BH; h < BH; h += s.fold_blocks - BH) copy_tail(s, h, tid);
      return;
    }
    bh = b;
    fold_head<F>(s, bh, smem, tid, s.fold_blocks == BH);
  } else {
    bh = attention_block<F, true, true>(a, b - s.fold_blocks, smem, zs, bad_flag);
  }
  __syncthreads();
  if (tid == 0) {
    // the fold workgroup releases xs (its threads' stores precede the barrier above); the
    // last workgroup acquires it
    const unsigned prev =
        b < s.fold_blocks
            ? __hip_atomic_fetch_add(s.counter + bh, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT)
            : __hip_atomic_fetch_add(s.counter + bh, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int last = prev == (unsigned)(s.per_head - 1) ? 1 : 0;
    if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    last_flag = last;
  }
  __syncthreads();
  if (!last_flag) return;
  finish_head<F>(s, bh, tid);
  if (tid == 0)   // ready for the next call
    __hip_atomic_store(s.counter + bh, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

int attn_bf16_tile_rows() { return QT; }

hipError_t launch_step_bf16(const AttnArgs& a, const StepArgs& s, int F, hipStream_t stream) {
  dim3 grid(s.fold_blocks + a.nblocks), block(NT);
  switch (F) {
    case 64:  hipLaunchKernelGGL(recurrent_step_bf16_kernel<64>, grid, block, 0, stream, a, s); break;
    case 128: hipLaunchKernelGGL(recurrent_step_bf16_kernel<128>, grid, block, 0, stream, a, s); break;
    case 256: hipLaunchKernelGGL(recurrent_step_bf16_kernel<256>, grid, block, 0, stream, a, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Compute units of the current device (one persistent attention workgroup each).
static int device_cus() {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cached[dev] = n;
  }
  return cached[dev];
}

// Query tiles per compute unit from which the persistent launch is used: with fewer, the
// hardware's own dispatch was faster (the 21x20x30 workload, 2.6 tiles per unit, lost
// 1.7 %; 12.5 and 14.1 tiles per unit gained 1.0 % and 3.9 %).
constexpr int kPersistentMinTiles = 4;

// Whether a launch of nblocks query tiles runs persistent (then a.queue must be set).
bool attn_bf16_persistent(int nblocks) {
  const int cus = device_cus();
  return cus > 0 && nblocks >= kPersistentMinTiles * cus;
}

hipError_t launch_attn_bf16(const AttnArgs& a, int F, hipStream_t stream) {
  const dim3 grid(a.queue ? device_cus() : a.nblocks), block(NT);
  if (grid.x == 0) return hipErrorInvalidDevice;
  if (a.queue) {
    switch (F) {
      case 64:  hipLaunchKernelGGL((hybrid_attn_bf16_kernel<64, true>), grid, block, 0, stream, a); break;
      case 128: hipLaunchKernelGGL((hybrid_attn_bf16_kernel<128, true>), grid, block, 0, stream, a); break;
      case 256: hipLaunchKernelGGL((hybrid_attn_bf16_kernel<256, true>), grid, block, 0, stream, a); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  switch (F) {
    case 64:  hipLaunchKernelGGL((hybrid_attn_bf16_kernel<64, false>), grid, block, 0, stream, a); break;
    case 128: hipLaunchKernelGGL((hybrid_attn_bf16_kernel<128, false>), grid, block, 0, stream, a); break;
    case 256: hipLaunchKernelGGL((hybrid_attn_bf16_kernel<256, false>), grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace rehyat
