// state_bf16.hip - linear-branch state on bf16 MFMA (gfx950), D = 128:
//   * per-segment partial sums  dS = phi(K_seg)^T V_seg  (F x D, fp32) and dz = sum phi(K_seg)
//     (the sums s_t, z_t of the chunk-wise RNN, papernotes.org ReHyAt note, key design 4);
//   * the feature map phi(x) = 1 + u + u^2/2, u = x W / sqrt(D), as a standalone op.
//
// U = K W is computed with K rows as the A operand (rows loaded in kappa order) and W^T
// as the B operand; its C tile has lane = feature and element i = key cidx(i, lane), which
// is exactly the A operand phi(K)^T of dS = phi(K)^T V. V enters as the B operand from
// the transposed V^T tile.
#include "tiles_bf16.h"

namespace rehyat {

namespace {

// F/32 feature blocks spread over 4 waves.
template <int F>
struct FBlocks {
  static constexpr int total = F / 32;
  static constexpr int per_wave = total >= 4 ? total / 4 : 1;
};

template <int F>
__global__ void __launch_bounds__(256)
state_partial_bf16_kernel(StateArgs a) {
  // W^T [F][128] (K-tile layout) + one K tile + one V^T tile
  __shared__ __attribute__((aligned(16))) unsigned char wt[F * 256];
  __shared__ __attribute__((aligned(16))) unsigned char kt[kKTileBytes];
  __shared__ __attribute__((aligned(16))) unsigned char vt[kVTileBytes];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int seg = blockIdx.x % a.n_seg;
  const int bh = blockIdx.x / a.n_seg;
  const int h = bh % a.H;
  const int64_t r0 = (int64_t)seg * a.seg_len;
  const int64_t r1 = (r0 + a.seg_len < a.n) ? r0 + a.seg_len : a.n;
  const int nrows = (int)(r1 - r0);

  const uint16_t* W = reinterpret_cast<const uint16_t*>(a.Wk) +
                      (a.w_per_head ? (int64_t)h * kDim * F : 0);
  stage_wt(wt, W, F, 0, F, tid);

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

  constexpr int PW = FBlocks<F>::per_wave;
  const bool active = wave < FBlocks<F>::total;
  f32x16 acc[PW][4];
  float zp[PW];
#pragma unroll
  for (int p = 0; p < PW; ++p) {
    zp[p] = 0.0f;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[p][db][i] = 0.0f;
  }

  const int ntiles = (nrows + kTileRows - 1) / kTileRows;
#pragma unroll 1
  for (int ti = 0; ti < ntiles; ++ti) {
    TileRegs r;
    tile_load(r, ks, vs, (int64_t)ti * kTileRows, tid);
    __syncthreads();   // previous tile fully consumed (and W^T staged on the first pass)
    tile_store(r, kt, vt, tid);
    __syncthreads();
    if (!active) continue;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key0 = ti * kTileRows + kb * 32;
      if (key0 >= nrows) break;
      const int arow = 32 * kb + kappa(lane & 31);
#pragma unroll
      for (int p = 0; p < PW; ++p) {
        const int fb = wave + 4 * p;
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
        zp[p] += zsum;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const int d = 32 * db + (lane & 31);
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            bf16x8 bv = as_bf16x8(lds_read16(vt, vtile_chunk_off(d, 4 * kb + 2 * j + (lane >> 5))));
            acc[p][db] = mfma32(Pk[j], bv, acc[p][db]);
          }
        }
      }
    }
  }

  if (!active) return;
  const int E = F * kDim + F;
  float* out = a.part + ((int64_t)bh * a.n_seg + seg) * E;
#pragma unroll
  for (int p = 0; p < PW; ++p) {
    const int fb = wave + 4 * p;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int d = 32 * db + (lane & 31);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int f = 32 * fb + crow(i, lane);
        out[(int64_t)f * kDim + d] = acc[p][db][i];
      }
    }
    const float zf = pair_sum(zp[p]);
    if (lane < 32) out[F * kDim + 32 * fb + lane] = zf;
  }
}

// phi(x) for rows of x: U = X W on MFMA, phi = 1 + u + u^2/2, stored as bf16 or fp32.
template <int F>
__global__ void __launch_bounds__(256)
phi_bf16_kernel(const uint16_t* x, int64_t n, const uint16_t* Wall, int w_per_head, int H,
                void* out, int out_f32, float u_scale, int tiles_per_head) {
  __shared__ __attribute__((aligned(16))) unsigned char wt[F * 256];
  __shared__ __attribute__((aligned(16))) unsigned char kt[kKTileBytes];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bh = blockIdx.x / tiles_per_head;
  const int ti = blockIdx.x % tiles_per_head;
  const int h = bh % H;
  const uint16_t* W = Wall + (w_per_head ? (int64_t)h * kDim * F : 0);
  stage_wt(wt, W, F, 0, F, tid);
  const uint16_t* xh = x + head_off(bh, n, kDim);
  const int64_t row0 = (int64_t)ti * kTileRows;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    int id = it * 256 + tid;
    int row = id >> 4, c = id & 15;
    u32x4 v = (row0 + row < n) ? *reinterpret_cast<const u32x4*>(xh + (row0 + row) * kDim + c * 8)
                               : u32x4{0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4*>(kt + ktile_off(row, c)) = v;
  }
  __syncthreads();
  constexpr int NFB = F / 32;
  // 2 row blocks x NFB feature blocks, spread over the 4 waves
  for (int job = wave; job < 2 * NFB; job += 4) {
    const int kb = job / NFB, fb = job % NFB;
    f32x16 U;
#pragma unroll
    for (int i = 0; i < 16; ++i) U[i] = 0.0f;
    const int arow = 32 * kb + kappa(lane & 31);
    const int brow = 32 * fb + (lane & 31);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int c = 2 * s + (lane >> 5);
      U = mfma32(as_bf16x8(lds_read16(kt, ktile_off(arow, c))),
                 as_bf16x8(lds_read16(wt, ktile_off(brow, c))), U);
    }
    const int f = 32 * fb + (lane & 31);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t row = row0 + 32 * kb + cidx(i, lane);
      if (row >= n) continue;
      float u = U[i] * u_scale;
      float p = 1.0f + u + 0.5f * u * u;
      const int64_t o = head_off(bh, n, F) + row * F + f;
      if (out_f32) reinterpret_cast<float*>(out)[o] = p;
      else reinterpret_cast<bf16*>(out)[o] = (bf16)p;
    }
  }
}

}  // namespace

hipError_t launch_state_partial_bf16(const StateArgs& a, int F, int BH, hipStream_t stream) {
  dim3 grid(BH * a.n_seg), block(256);
  switch (F) {
    case 64:  hipLaunchKernelGGL(state_partial_bf16_kernel<64>, grid, block, 0, stream, a); break;
    case 128: hipLaunchKernelGGL(state_partial_bf16_kernel<128>, grid, block, 0, stream, a); break;
    case 256: hipLaunchKernelGGL(state_partial_bf16_kernel<256>, grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_phi_bf16(const void* x, int64_t n, const void* W, int w_per_head, int H, int BH,
                           int F, void* out, int out_f32, float u_scale, hipStream_t stream) {
  const int tph = (int)((n + kTileRows - 1) / kTileRows);
  dim3 grid(BH * tph), block(256);
  const uint16_t* xx = reinterpret_cast<const uint16_t*>(x);
  const uint16_t* ww = reinterpret_cast<const uint16_t*>(W);
  switch (F) {
    case 64:  hipLaunchKernelGGL(phi_bf16_kernel<64>, grid, block, 0, stream, xx, n, ww, w_per_head, H, out, out_f32, u_scale, tph); break;
    case 128: hipLaunchKernelGGL(phi_bf16_kernel<128>, grid, block, 0, stream, xx, n, ww, w_per_head, H, out, out_f32, u_scale, tph); break;
    case 256: hipLaunchKernelGGL(phi_bf16_kernel<256>, grid, block, 0, stream, xx, n, ww, w_per_head, H, out, out_f32, u_scale, tph); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace rehyat
