// partial_bf16.h - partial state sums of one row segment on bf16 MFMA (gfx950), D = 128:
//   dS = phi(K_seg)^T V_seg (F x D, fp32) and dz = sum phi(K_seg), phi(x) = 1 + u + u^2/2,
//   u = x W / sqrt(D)
// (the sums s_t, z_t of the chunk-wise RNN, papernotes.org ReHyAt note, key design 4).
// The state kernel (one segment per workgroup of 4 waves) streams 32-row tiles of K and V
// into LDS stages by direct-to-LDS loads (partial_issue) and reduces every tile with
// partial_tile; the fold workgroup of the single-launch recurrent step (two segments per
// 512-thread workgroup) stages 64-row tiles through registers (segment_sums). Both take the
// same operand values in the same MFMA chain order, so they produce the same bits.
//
// U = K W is computed with K rows as the A operand (rows read in kappa order) and W^T as
// the B operand, held in registers; its C tile has lane = feature and element i = key
// cidx(i, lane), which is exactly the A operand phi(K)^T of dS = phi(K)^T V. V enters as
// the B operand through transposing reads of the row-major V tile.
#pragma once

#include "tiles_bf16.h"

namespace rehyat {

// F/32 feature blocks spread over 4 waves.
template <int F>
struct FBlocks {
  static constexpr int total = F / 32;
  static constexpr int per_wave = total >= 4 ? total / 4 : 1;
};

// Rows of segment seg: [seg * seg_len, min(+seg_len, n)).
__device__ __forceinline__ int segment_rows(const StateArgs& a, int seg) {
  const int64_t r0 = (int64_t)seg * a.seg_len;
  const int64_t r1 = (r0 + a.seg_len < a.n) ? r0 + a.seg_len : a.n;
  return (int)(r1 - r0);
}

// ---- register-staged 64-row tiles (the fold workgroup of the single-launch step) ----
// The same values and MFMA chains as partial_tile over the segment's 32-row tiles, so the
// fold and the state kernel produce the same bits.
// LDS of one segment's tiles (K tile + V^T tile); W^T takes F * 256 more.
constexpr int kPartialTileBytes = kKTileBytes + kVTileBytes;

__device__ __forceinline__ int segment_tiles(const StateArgs& a, int seg) {
  return (segment_rows(a, seg) + kTileRows - 1) / kTileRows;
}

// Partial sums of segment seg of head bh, left in registers (acc, zp) of 256 threads
// (tid 0..255) that own the tiles kt, vt. W^T of the head ([F][128], K-tile layout) is in
// wt, or is being staged there by the workgroup before this call: the loop's first barrier
// orders it. ntiles: iterations of the tile loop; every thread of the workgroup passes the
// same value (the loop holds barriers), at least segment_tiles(a, seg). seg < 0: no segment
// (the threads only take part in the barriers). Element i of acc[p][db] of lane l is
// dS[32 fb + crow(i, l)][32 db + l mod 32], fb = wave + 4 p; the pair sum of zp[p] is
// dz[32 fb + l mod 32].
// Split form (kPart >= 0, F = 256): the 256 threads take the feature blocks 4 kPart ..
// 4 kPart + 3 only (one per wave), so that two groups of 256 threads form one segment's
// partial together with half the accumulators each.
template <int F, int kPart = -1>
struct PartialShape {
  static constexpr int PW = kPart >= 0 ? 1 : FBlocks<F>::per_wave;   // blocks per wave
  __device__ static int fb(int wave, int p) { return kPart >= 0 ? 4 * kPart + wave : wave + 4 * p; }
};

template <int F, int kPart = -1>
struct PartialRegs {
  f32x16 acc[PartialShape<F, kPart>::PW][4];
  float zp[PartialShape<F, kPart>::PW];
};

template <int F, int kPart = -1>
__device__ __forceinline__ bool partial_active(int seg, int tid) {
  return PartialShape<F, kPart>::fb(tid >> 6, 0) < FBlocks<F>::total && seg >= 0;
}

template <int F, int kPart = -1>
__device__ __forceinline__ void segment_sums(PartialRegs<F, kPart>& R, const StateArgs& a,
                                             int bh, int seg, int ntiles,
                                             const unsigned char* wt, unsigned char* kt,
                                             unsigned char* vt, int tid) {
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t r0 = (int64_t)(seg < 0 ? 0 : seg) * a.seg_len;
  const int nrows = seg < 0 ? 0 : segment_rows(a, seg);

  // Rows of this segment: global row r0 + w.
  RowSrc ks, vs;
  {
    const uint16_t* ka = reinterpret_cast<const uint16_t*>(a.ka) + head_off(bh, a.a_rows, kDim);
    const uint16_t* va = reinterpret_cast<const uint16_t*>(a.va) + head_off(bh, a.a_rows, kDim);
    const uint16_t* kb = reinterpret_cast<const uint16_t*>(a.kb) + head_off(bh, a.b_rows, kDim);
    const uint16_t* vb = reinterpret_cast<const uint16_t*>(a.vb) + head_off(bh, a.b_rows, kDim);
    // window-relative row w -> global row r0 + w; A covers global rows [0, na)
    const int64_t na_rel = (a.na - r0) > 0 ? (a.na - r0) : 0;
    ks = RowSrc{ka, kb + (r0 > a.na ? (r0 - a.na) * kDim : 0) + a.b_row0 * kDim,
                a.a_row0 + r0, na_rel, (int64_t)nrows};
    vs = RowSrc{va, vb + (r0 > a.na ? (r0 - a.na) * kDim : 0) + a.b_row0 * kDim,
                a.a_row0 + r0, na_rel, (int64_t)nrows};
  }

  constexpr int PW = PartialShape<F, kPart>::PW;
  const bool active = partial_active<F, kPart>(seg, tid);
#pragma unroll
  for (int p = 0; p < PW; ++p) {
    R.zp[p] = 0.0f;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) R.acc[p][db][i] = 0.0f;
  }

  TileRegs r;
  tile_load(r, ks, vs, 0, tid);
#pragma unroll 1
  for (int ti = 0; ti < ntiles; ++ti) {
    __syncthreads();   // previous tile fully consumed (and W^T staged on the first pass)
    tile_store(r, kt, vt, tid);
    // the next tile's global loads fly while this tile is reduced
    if (ti + 1 < ntiles) tile_load(r, ks, vs, (int64_t)(ti + 1) * kTileRows, tid);
    __syncthreads();
    if (!active) continue;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key0 = ti * kTileRows + kb * 32;
      if (key0 >= nrows) break;
      const int arow = 32 * kb + kappa(lane & 31);
#pragma unroll
      for (int p = 0; p < PW; ++p) {
        const int fb = PartialShape<F, kPart>::fb(wave, p);
        f32x16 U;
#pragma unroll
        for (int i = 0; i < 16; ++i) U[i] = 0.0f;
        const int brow = 32 * fb + (lane & 31);
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const int c = 2 * s + (lane >> 5);
          bf16x8 av = as_bf16x8(lds_read16(kt, ktile_off(arow, c)));
          bf16x8 bv = as_bf16x8(lds_read16(wt, ktile_off(brow, c)));
          U = mfma32(av, bv, U);
        }
        bf16x8 Pk[2];
        float zsum = 0.0f;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          u32x4 pk;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i0 = 8 * j + 2 * e;
            const int key = key0 + cidx(i0, lane);
            float u0 = U[i0] * a.u_scale, u1 = U[i0 + 1] * a.u_scale;
            float p0 = (key < nrows) ? 1.0f + u0 + 0.5f * u0 * u0 : 0.0f;
            float p1 = (key + 1 < nrows) ? 1.0f + u1 + 0.5f * u1 * u1 : 0.0f;
            unsigned w = pack_bf16_u32(p0, p1);
            zsum += bf16_lo(w) + bf16_hi(w);
            pk[e] = w;
          }
          Pk[j] = as_bf16x8(pk);
        }
        R.zp[p] += zsum;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const int d = 32 * db + (lane & 31);
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            bf16x8 bv = as_bf16x8(lds_read16(vt, vtile_chunk_off(d, 4 * kb + 2 * j + (lane >> 5))));
            R.acc[p][db] = mfma32(Pk[j], bv, R.acc[p][db]);
          }
        }
      }
    }
  }
}

// Visit every element of a partial held by this thread: fn(offset in [F*128 + F], value),
// dS entries at f * 128 + d, dz entries at F * 128 + f (the z sums from lanes < 32).
template <int F, int kPart = -1, typename Fn>
__device__ __forceinline__ void for_partial(const PartialRegs<F, kPart>& R, int tid, Fn fn) {
  const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int p = 0; p < PartialShape<F, kPart>::PW; ++p) {
    const int fb = PartialShape<F, kPart>::fb(wave, p);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int d = 32 * db + (lane & 31);
#pragma unroll
      for (int i = 0; i < 16; ++i) fn((32 * fb + crow(i, lane)) * kDim + d, R.acc[p][db][i]);
    }
    const float zf = pair_sum(R.zp[p]);
    if (lane < 32) fn(F * kDim + 32 * fb + lane, zf);
  }
}

// ---- direct-to-LDS 32-row tiles (the state kernel) --------------------------------
// Tiles of 32 rows in LDS. K slot u of the 9 KB K region holds row u / 17, chunk u % 17
// (rows of 272 B: the 16-byte pad slot takes a copy of chunk 0; the slots past 32 rows hold
// rows of the next tile, unused); V slot u of the V region holds row u / 18, chunk u % 18
// (rows of 288 B, pad slots 16 and 17 copy chunk 0). Rows past the segment come back as
// zeros from the descriptor's range.
constexpr int kPRows = 32;                    // rows per tile
constexpr int kPKRow = 272;                   // K row: 256 B + 16 B pad
constexpr int kPVRow = 288;                   // V row: 256 B + 32 B pad
constexpr int kPInsts = 9;                    // 1 KB DMA instructions per tile and tensor
constexpr int kPRegion = kPInsts * 1024;      // 9 KB each for K and V
constexpr int kPStage = 2 * kPRegion;         // 18 KB

// This wave's direct-to-LDS loads of tile t (rows 32 t ..) of the segment whose K and V
// rows the descriptors kr, vr cover, into the stage at LDS address st: instructions
// j = wave + kWaves i of the tile's 2 * kPInsts.
template <int kWaves>
__device__ __forceinline__ void partial_issue(i32x4 kr, i32x4 vr, unsigned st, int t, int wave,
                                              int lane) {
#pragma unroll
  for (int i = 0; i < (2 * kPInsts + kWaves - 1) / kWaves; ++i) {
    const int j = wave + kWaves * i;
    if (j < kPInsts) {
      const int u = 64 * j + lane;
      const int r = u / 17;
      int c = u - 17 * r;
      c = c == 16 ? 0 : c;
      dma16(kr, st + j * 1024, (t * kPRows + r) * 256 + c * 16);
    } else if (j < 2 * kPInsts) {
      const int jj = j - kPInsts;
      const int u = 64 * jj + lane;
      const int r = u / 18;
      int c = u - 18 * r;
      c = c >= 16 ? 0 : c;
      dma16(vr, st + kPRegion + jj * 1024, (t * kPRows + r) * 256 + c * 16);
    }
  }
}

// Loads one wave issues per tile in partial_issue<kWaves>.
template <int kWaves>
__device__ __forceinline__ int partial_insts(int wave) {
  return (2 * kPInsts - wave + kWaves - 1) / kWaves;
}

// One 32-row tile (rows key0 .. key0 + 31 of a segment of nrows rows) for feature block fb
// of this wave and the NDB value blocks db0 .. db0 + NDB - 1: U = K W (wf: W^T rows
// 32 fb + l % 32 as B operand fragments), p = phi(U) rounded to bf16 (zero past nrows),
// zp += sum of this lane's p, acc[i] += P^T V[:, 32 (db0 + i) ..]. Element i of acc[b] of
// lane l is dS[32 fb + crow(i, l)][32 (db0 + b) + l mod 32]; the pair sum of zp over all
// tiles is dz[32 fb + l mod 32].
template <int NDB>
__device__ __forceinline__ void partial_tile(const unsigned char* kt, const unsigned char* vt,
                                             const bf16x8 (&wf)[8], int key0, int nrows,
                                             float u_scale, int db0, int lane,
                                             f32x16 (&acc)[NDB], float& zp) {
  f32x16 U;
#pragma unroll
  for (int i = 0; i < 16; ++i) U[i] = 0.0f;
  const int arow = kappa(lane & 31);
  bf16x8 kf[8];
#pragma unroll
  for (int s = 0; s < 8; ++s)
    kf[s] = as_bf16x8(lds_read16(kt, arow * kPKRow + (2 * s + (lane >> 5)) * 16));
#pragma unroll
  for (int s = 0; s < 8; ++s) U = mfma32(kf[s], wf[s], U);
  bf16x8 Pk[2];
  float zsum = 0.0f;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    u32x4 pk;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i0 = 8 * j + 2 * e;
      const int key = key0 + cidx(i0, lane);
      float u0 = U[i0] * u_scale, u1 = U[i0 + 1] * u_scale;
      float p0 = (key < nrows) ? 1.0f + u0 + 0.5f * u0 * u0 : 0.0f;
      float p1 = (key + 1 < nrows) ? 1.0f + u1 + 0.5f * u1 * u1 : 0.0f;
      unsigned w = pack_bf16_u32(p0, p1);
      zsum += bf16_lo(w) + bf16_hi(w);
      pk[e] = w;
    }
    Pk[j] = as_bf16x8(pk);
  }
  zp += zsum;
  bf16x8 vf[NDB][2];
#pragma unroll
  for (int b = 0; b < NDB; ++b)
#pragma unroll
    for (int j = 0; j < 2; ++j) vf[b][j] = frag_tr(vt, kPVRow, 16 * j, 32 * (db0 + b), lane);
#pragma unroll
  for (int b = 0; b < NDB; ++b)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[b] = mfma32(Pk[j], vf[b][j], acc[b]);
}

// W^T rows 32 fb + l % 32 (staged in the K-tile layout at wt) as the B operand fragments
// of U = K W.
__device__ __forceinline__ void partial_wt_frags(bf16x8 (&wf)[8], const unsigned char* wt,
                                                 int fb, int lane) {
#pragma unroll
  for (int s = 0; s < 8; ++s)
    wf[s] = as_bf16x8(lds_read16(wt, ktile_off(32 * fb + (lane & 31), 2 * s + (lane >> 5))));
}

}  // namespace rehyat
