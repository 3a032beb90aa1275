// bwd_bf16.hip - backward of the non-recursive (training-time) causal form of ReHyAt hybrid
// attention, bf16 inputs, D = 128, the fixed feature map phi = 1 + u + u^2/2, u = x W/sqrt(D)
// (papernotes.org note "ReHyAt: Recurrent Hybrid Attention for Video Diffusion
// Transformers", method details, key designs 1 and 4).
//
// For query i with weights w_ij (exp(q_i.k_j/sqrt(D)) on its softmax window, phi(q_i).phi(k_j)
// on its linear set) and den_i = sum_j w_ij, y_i = sum_j w_ij v_j / den_i. With upstream dy:
//   dL/dw_ij = g_i.v_j - c_i,   g_i = dy_i / den_i,   c_i = (dy_i . y_i) / den_i;
//   window:  ds_ij = w_ij dL/dw_ij = p_ij (dy_i.v_j - dy_i.y_i), p_ij = w_ij / den_i
//            dq_i += sum_j ds_ij k_j / sqrt(D),  dk_j += sum_i ds_ij q_i / sqrt(D),
//            dv_j += sum_i p_ij dy_i;
//   linear:  dphi(q_i) = S_t g_i - c_i z_t           (S_t, z_t: the chunk's forward state)
//            dphi(k_j) = G_j v_j - h_j,  dv_j += G_j^T phi(k_j),
//            G_j = sum_{i: j in L_i} phi(q_i) g_i^T,  h_j = sum_i phi(q_i) c_i
//            (the reverse state: for causal sets a suffix over the chunks after j's window);
//   map:     gx = dphi (1 + u) / sqrt(D),  dx += W gx,  dW += sum_rows x gx^T.
// den comes from the forward as lse = log2(den). MFMA operands follow the conventions of
// common.h (C tiles of a first product taken in the kappa row order feed the next product
// directly). The window parts' tiles are stored in bank-conflict-free swizzled layouts
// (Swz320, Swz256 below); the linear parts' slabs in rows of 128 bf16 padded to 272 bytes.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "common.h"
#include "tiles_bf16.h"


namespace rehyat {
namespace {

constexpr int kRowB = 272;                     // LDS row of 128 bf16 + 16 B pad

__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0070); }

// Operand tiles of the window parts. Their rows (128 bf16: one query, key or value each)
// are read two ways: as 16-byte A-operand pieces, 16 rows (in kappa order) at one chunk per
// 16 lanes, which LDS serves in one 256-byte pass; and by the transposing read, whose 32
// lanes of a pass touch 4 consecutive rows x 64 bytes. No padded row stride alone keeps
// both on 64 distinct banks (272 B serves the first and costs the second four passes), so
// chunk c (16 bytes) of row r is stored at chunk c ^ h(r mod 16) of the row:
//   Swz320: rows of 320 B (80 words, 16 mod 64; slots 16..19 are pad), h = (r / 4) mod 4;
//   Swz256: rows of 256 B, h = (r ^ 4r) mod 16.
// Either way every pass of both reads hits 64 distinct banks. a_off and t_off are the byte
// offsets of a lane's pieces within a block of 32 (A pieces) or 16 (transposing reads) rows;
// they are written so that few distinct per-lane bases remain (the rest are immediates):
// Swz320's h leaves chunk bits 2, 3 alone (2 + 2 bases); in Swz256 row r + 4 has h ^ 4, so the
// second transposing read of a fragment is the first one's of column block db ^ 1, four rows
// down (8 + 4 bases). The 256-byte form is for the tile pairs that do not fit at 320 B.
struct Swz320 {
  static constexpr int kRow = 320, kSlots = 20;
  __device__ static int h(int r) { return (r >> 2) & 3; }
  // A piece s (chunk 2s + l/32) of row kappa(l mod 32)
  __device__ static int a_off(int lane, int s) {
    const int r = kappa(lane & 31);
    return r * kRow + 16 * ((2 * (s & 1) + (lane >> 5)) ^ h(r)) + 64 * (s >> 1);
  }
  // transposing read hi (rows 4 hi .. 4 hi + 3 of each 8) of columns 32 db .. 32 db + 31
  __device__ static int t_off(int lane, int db, int hi) {
    const int g = lane >> 4, q = lane & 15;
    const int r = 8 * (g >> 1) + (q >> 2) + 4 * hi;
    return r * kRow + 16 * ((2 * (g & 1) + ((q & 3) >> 1)) ^ h(r)) + 8 * (q & 1) + 64 * db;
  }
};
struct Swz256 {
  static constexpr int kRow = 256, kSlots = 16;
  __device__ static int h(int r) { return (r ^ (r << 2)) & 15; }
  __device__ static int a_off(int lane, int s) {
    const int r = kappa(lane & 31);
    return r * kRow + 16 * ((2 * s + (lane >> 5)) ^ h(r));
  }
  __device__ static int t_off(int lane, int db, int hi) {
    const int g = lane >> 4, q = lane & 15;
    const int r = 8 * (g >> 1) + (q >> 2);
    const int d = hi ? db ^ 1 : db;
    return (r + 4 * hi) * kRow + 16 * ((4 * d + 2 * (g & 1) + ((q & 3) >> 1)) ^ h(r)) + 8 * (q & 1);
  }
};

// Direct-to-LDS copy of ROWS rows of 256 B (row r at byte r*256 of the buffer) into a tile
// of layout L at LDS address dst. Instruction j writes the 64 consecutive 16-byte slots
// 64j..64j+63; slot u is row u / kSlots, stored chunk p = u mod kSlots, which holds chunk
// p ^ h(row) (pad slots take a copy of chunk 0). Rows past the buffer's range read as
// zeros. The loads are ones the compiler does not track (tiles_bf16.h, dma16), so it places
// no wait for them before later LDS reads: the caller waits (vmcnt) before the barrier
// that hands the tile over.
template <class L, int ROWS, int NW>
__device__ __forceinline__ void dma_tile(i32x4 src, unsigned dst, int wave, int lane) {
  constexpr int kInsts = ROWS * L::kSlots / 64;
  static_assert(ROWS * L::kSlots % 64 == 0, "whole DMA instructions");
#pragma unroll
  for (int i = 0; i < (kInsts + NW - 1) / NW; ++i) {
    const int j = wave + NW * i;
    if (j < kInsts) {
      const int u = 64 * j + lane;
      const int r = u / L::kSlots;
      const int p = u - L::kSlots * r;
      const int c = p < 16 ? p ^ L::h(r & 15) : 0;
      dma16(src, dst + j * 1024, r * 256 + c * 16);
    }
  }
}

// Transposing fragment of a layout-L tile: the two reads at lo and hi (t_off(.., 0 / 1)).
__device__ __forceinline__ bf16x8 frag_tr_at(const unsigned char* lo, const unsigned char* hi) {
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)lo);
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)hi);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Plain staging of `rows` rows of `cols` bf16 (row stride ld elements, from column c0) into
// LDS rows of `rb` bytes, by `nthr` threads.
__device__ __forceinline__ void stage_rows(unsigned char* dst, int rb, const uint16_t* src,
                                           int64_t ld, int c0, int rows, int cols, int tid,
                                           int nthr) {
  const int cpr = cols / 8;
  for (int id = tid; id < rows * cpr; id += nthr) {
    const int r = id / cpr, c = id - r * cpr;
    *reinterpret_cast<u32x4*>(dst + r * rb + 16 * c) =
        *reinterpret_cast<const u32x4*>(src + r * ld + c0 + 8 * c);
  }
}

// ---- per-row preparation ----------------------------------------------------------------
// 16 lanes per row (8 elements each): dy.y, 2^-lse, and the bf16 rows of dy and dy / den.
// dvec holds (dy.y) / sqrt(D) (us = 1/sqrt(D)), the form in which the window parts use it:
// ds = p (dP - dy.y) / sqrt(D) = p * fma(dP, us, -dvec).
__global__ void __launch_bounds__(256)
bwd_prep_kernel(const void* __restrict__ y, const void* __restrict__ dy, int y_f32,
                const float* __restrict__ lse, int64_t rows, float us, uint16_t* __restrict__ dyb,
                uint16_t* __restrict__ gb, float* __restrict__ cvec, float* __restrict__ dvec) {
  const int tid = threadIdx.x;
  const int64_t row = (int64_t)blockIdx.x * 16 + (tid >> 4);
  const int c = tid & 15;
  const bool ok = row < rows;
  const int64_t off = (ok ? row : 0) * kDim + 8 * c;
  float yv[8], gv[8];
  if (y_f32) {
    const f32x4* yp = reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(y) + off);
    const f32x4* gp = reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(dy) + off);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f32x4 a = yp[h], b = gp[h];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        yv[4 * h + e] = a[e];
        gv[4 * h + e] = b[e];
      }
    }
  } else {
    const u32x4 a = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(y) + off);
    const u32x4 b = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(dy) + off);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      yv[2 * e] = bf16_lo(a[e]);
      yv[2 * e + 1] = bf16_hi(a[e]);
      gv[2 * e] = bf16_lo(b[e]);
      gv[2 * e + 1] = bf16_hi(b[e]);
    }
  }
  float dot = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) dot = fmaf(gv[e], yv[e], dot);
  dot += __shfl_xor(dot, 1);
  dot += __shfl_xor(dot, 2);
  dot += __shfl_xor(dot, 4);
  dot += __shfl_xor(dot, 8);
  if (!ok) return;
  const float inv = fast_exp2(-lse[row]);
  u32x4 pd, pg;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    pd[e] = pack_bf16_u32(gv[2 * e], gv[2 * e + 1]);
    pg[e] = pack_bf16_u32(gv[2 * e] * inv, gv[2 * e + 1] * inv);
  }
  *reinterpret_cast<u32x4*>(dyb + row * kDim + 8 * c) = pd;
  *reinterpret_cast<u32x4*>(gb + row * kDim + 8 * c) = pg;
  if (c == 0) {
    cvec[row] = dot * inv;
    dvec[row] = dot * us;
  }
}

// ---- state rows to bf16 ------------------------------------------------------------------
// nst states per head (state (bh, t) at S + bh*s_bh + t*s_t, [F][128] fp32) to bf16 rows at
// img + (bh*nst + t)*F*128.
__global__ void __launch_bounds__(256)
state_rows_bf16_kernel(const float* __restrict__ S, int64_t s_bh, int64_t s_t, int nst, int F,
                       uint16_t* __restrict__ img) {
  const int u = blockIdx.x * 256 + threadIdx.x;   // 8 elements per unit
  const int t = blockIdx.y, bh = blockIdx.z;
  if (u >= F * kDim / 8) return;
  const float* src = S + (int64_t)bh * s_bh + (int64_t)t * s_t + u * 8;
  const f32x4 a = reinterpret_cast<const f32x4*>(src)[0];
  const f32x4 b = reinterpret_cast<const f32x4*>(src)[1];
  u32x4 w;
  w[0] = pack_bf16_u32(a[0], a[1]);
  w[1] = pack_bf16_u32(a[2], a[3]);
  w[2] = pack_bf16_u32(b[0], b[1]);
  w[3] = pack_bf16_u32(b[2], b[3]);
  *reinterpret_cast<u32x4*>(img + ((int64_t)bh * nst + t) * F * kDim + u * 8) = w;
}

// W [nW][128][F] -> W^T [nW][F][128], bf16.
__global__ void __launch_bounds__(256)
transpose_w_kernel(const uint16_t* __restrict__ W, int F, uint16_t* __restrict__ Wt) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  const int h = blockIdx.y;
  if (e >= F * kDim) return;
  const int f = e / kDim, d = e - f * kDim;
  Wt[(int64_t)h * F * kDim + e] = W[(int64_t)h * kDim * F + (int64_t)d * F + f];
}

// Reverse states of the causal sets. part [BH][T][E]: per query frame, the sums
// phi(q) g^T (F x 128) and phi(q) c (F). out [BH][T][E]: for key frame f, the sum over the
// query frames of every chunk whose causal linear set holds frame f, i.e. chunks t with
// lo_t >= (f + 1) HW, which start at frame F0(f) = Tc * ceil((f + 1 + To) / Tc).
__global__ void __launch_bounds__(256)
suffix_states_kernel(const float* __restrict__ part, float* __restrict__ out, int E, int T,
                     int Tc, int To) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  const int bh = blockIdx.y;
  if (e >= E) return;
  const float* p = part + (int64_t)bh * T * E + e;
  float* o = out + (int64_t)bh * T * E + e;
  float acc = 0.0f;
  int fs = T;   // acc = sum of part over frames [fs, T)
  for (int f = T - 1; f >= 0; --f) {
    const int f0 = Tc * ((f + 1 + To + Tc - 1) / Tc);
    for (; fs > f0; --fs) acc += p[(int64_t)(fs - 1) * E];
    o[(int64_t)f * E] = acc;
  }
}

// Per-head dW^T sums [BH][F][128] (stride E) -> dW [nW][128][F]: summed over the batch for
// per-head maps (nW = H), over every head and batch item for a shared map (nW = 1).
__global__ void __launch_bounds__(256)
dw_finalize_kernel(const float* __restrict__ parts, int64_t E, int BH, int H, int per_head, int F,
                   float* __restrict__ dW) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  const int h = blockIdx.y;
  if (e >= kDim * F) return;
  const int d = e / F, f = e - d * F;
  float acc = 0.0f;
  for (int bh = per_head ? h : 0; bh < BH; bh += per_head ? H : 1)
    acc += parts[(int64_t)bh * E + (int64_t)f * kDim + d];
  dW[(int64_t)h * kDim * F + e] = acc;
}

// ---- dq: one workgroup of 8 waves per 256 queries of a chunk, lane = query ---------------
//
// Linear part (chunks with a non-empty causal linear set), per 128-feature slab: U^T = W^T
// Q^T and (S_t g)^T on MFMA (rows of W^T and of the state in kappa order, so the results are
// B operands over features), phi, dphi = S_t g - c z_t, gq = dphi (1 + u) / sqrt(D), and
// dq^T += W gq^T. Window part, per 32-key block: S^T = K Q^T, dP^T = V dY^T, p and ds in
// registers, dq^T += K^T ds^T with K^T read by the transposing LDS read.
constexpr int kQW = 8;                                   // waves of the dq kernel
constexpr int kLinLds = 3 * 128 * kRowB;                 // W^T, S and W slabs
constexpr int kKeyTile = 64;
using KL = Swz320;                                       // layout of the K and V tiles
constexpr int kDqLds = kLinLds > 4 * kKeyTile * KL::kRow ? kLinLds : 4 * kKeyTile * KL::kRow;

struct BwdGeo {
  int bh, t;
  int64_t row0;    // first row of the chunk
  int rows;        // rows of the chunk
  int64_t lo, hi;  // softmax window
};

__device__ __forceinline__ BwdGeo bwd_geo(const BwdArgs& a, int b, int& tile) {
  BwdGeo g;
  g.bh = b / a.tiles_per_head;
  const int r = b - g.bh * a.tiles_per_head;
  const int full = (a.n_chunks - 1) * a.tiles_per_chunk;
  if (r < full) {
    g.t = r / a.tiles_per_chunk;
    tile = r - g.t * a.tiles_per_chunk;
  } else {
    g.t = a.n_chunks - 1;
    tile = r - full;
  }
  const int64_t Np = (int64_t)a.Tc * a.HW;
  g.row0 = g.t * Np;
  g.rows = (int)((g.row0 + Np < a.N) ? Np : a.N - g.row0);
  g.lo = g.row0 - (int64_t)a.To * a.HW > 0 ? g.row0 - (int64_t)a.To * a.HW : 0;
  g.hi = g.row0 + g.rows;
  return g;
}

template <int F>
__global__ void __launch_bounds__(64 * kQW)
bwd_dq_kernel(BwdArgs a) {
  constexpr int FS = F < 128 ? F : 128;
  constexpr int RW = 2 * FS + 16;                        // bytes per W slab row
  __shared__ __attribute__((aligned(16))) unsigned char smem[kDqLds];
  __shared__ float zs[F];
  // the wave index is uniform: held in a scalar register, the tile loads' LDS addresses are
  // scalar too and free vector registers for the loop
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int qt;
  const BwdGeo g = bwd_geo(a, blockIdx.x, qt);
  const int qw0 = qt * 256 + wave * 32;                  // first query of the wave in the chunk
  const bool active = qw0 < g.rows;
  const int ql = qw0 + (lane & 31);
  const bool ok = active && ql < g.rows;
  const int64_t row = g.row0 + (ok ? ql : 0);            // this lane's query row
  const int64_t hrow = (int64_t)g.bh * a.N;              // head's first row
  const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + (hrow + row) * kDim + 8 * (lane >> 5);
  bf16x8 Qf[8];
#pragma unroll
  for (int s = 0; s < 8; ++s)
    Qf[s] = as_bf16x8(ok ? *reinterpret_cast<const u32x4*>(qp + 16 * s) : u32x4{0u, 0u, 0u, 0u});
  const float lse_l = ok ? a.lse[hrow + row] : 1.0e30f;
  const float dd_l = ok ? a.dvec[hrow + row] : 0.0f;
  const float c_l = ok ? a.cvec[hrow + row] : 0.0f;
  const float us = a.u_scale;
  f32x16 dQ[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dQ[db][i] = 0.0f;

  const int h = g.bh % a.H;
  uint16_t* phio = a.phi_out + (hrow + row) * F;
  uint16_t* go = a.g_out + (hrow + row) * F;
  if (g.lo > 0) {
    // ---- linear part ----
    bf16x8 Gf[8];
    {
      const uint16_t* gp = a.gb + (hrow + row) * kDim + 8 * (lane >> 5);
#pragma unroll
      for (int s = 0; s < 8; ++s)
        Gf[s] = as_bf16x8(ok ? *reinterpret_cast<const u32x4*>(gp + 16 * s) : u32x4{0u, 0u, 0u, 0u});
    }
    const uint16_t* wt = a.wt + (a.w_per_head ? (int64_t)h * F * kDim : 0);
    const uint16_t* w = a.w + (a.w_per_head ? (int64_t)h * kDim * F : 0);
    const uint16_t* simg = a.st_img + ((int64_t)g.bh * a.nslot + g.t) * F * kDim;
    const float* zsrc = a.st + ((int64_t)g.bh * a.nslot + g.t) * ((int64_t)F * kDim + F) + F * kDim;
    unsigned char* sWt = smem;
    unsigned char* sS = smem + 128 * kRowB;
    unsigned char* sW = smem + 2 * 128 * kRowB;
    for (int f = tid; f < F; f += 64 * kQW) zs[f] = zsrc[f];
    const int ab = kappa(lane & 31) * kRowB + 16 * (lane >> 5);   // A rows in kappa order
#pragma unroll 1
    for (int f0 = 0; f0 < F; f0 += FS) {
      __syncthreads();
      stage_rows(sWt, kRowB, wt + (int64_t)f0 * kDim, kDim, 0, FS, kDim, tid, 64 * kQW);
      stage_rows(sS, kRowB, simg + (int64_t)f0 * kDim, kDim, 0, FS, kDim, tid, 64 * kQW);
      stage_rows(sW, RW, w, F, f0, kDim, FS, tid, 64 * kQW);
      __syncthreads();
      if (!active) continue;
#pragma unroll 1
      for (int fb = 0; fb < FS / 32; ++fb) {
        f32x16 U, P1;
#pragma unroll
        for (int i = 0; i < 16; ++i) U[i] = P1[i] = 0.0f;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          U = mfma32(as_bf16x8(lds_read16(sWt, ab + fb * 32 * kRowB + 32 * s)), Qf[s], U);
          P1 = mfma32(as_bf16x8(lds_read16(sS, ab + fb * 32 * kRowB + 32 * s)), Gf[s], P1);
        }
        bf16x8 gqb[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          u32x4 pp, pg;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float ph2[2], gq2[2];
#pragma unroll
            for (int q2 = 0; q2 < 2; ++q2) {
              const int i = 8 * j + 2 * e + q2;
              const int f = f0 + 32 * fb + cidx(i, lane);
              const float u = U[i] * us;
              ph2[q2] = 1.0f + u + 0.5f * u * u;
              gq2[q2] = (P1[i] - c_l * zs[f]) * (1.0f + u) * us;
            }
            pp[e] = pack_bf16_u32(ph2[0], ph2[1]);
            pg[e] = pack_bf16_u32(gq2[0], gq2[1]);
          }
          gqb[j] = as_bf16x8(pg);
          const int fo = f0 + 32 * fb + 16 * j + 8 * (lane >> 5);
          if (ok) {
            *reinterpret_cast<u32x4*>(phio + fo) = pp;
            *reinterpret_cast<u32x4*>(go + fo) = pg;
          }
        }
        // dq^T += W gq^T: A = W rows d (lane % 32) at features 32 fb + 16 j + 8 (l / 32)
        const int wb = (lane & 31) * RW + 2 * (32 * fb + 8 * (lane >> 5));
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            dQ[db] = mfma32(as_bf16x8(lds_read16(sW, wb + db * 32 * RW + 32 * j)), gqb[j], dQ[db]);
      }
    }
  } else if (ok) {
    // no linear set: zero phi(q) and gq rows (they enter sums over every row later)
    for (int f = 8 * (lane >> 5); f < F; f += 16) {
      *reinterpret_cast<u32x4*>(phio + f) = u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(go + f) = u32x4{0u, 0u, 0u, 0u};
    }
  }

  // ---- window part ----
  bf16x8 DYf[8];
  {
    const uint16_t* dp = a.dyb + (hrow + row) * kDim + 8 * (lane >> 5);
#pragma unroll
    for (int s = 0; s < 8; ++s)
      DYf[s] = as_bf16x8(ok ? *reinterpret_cast<const u32x4*>(dp + 16 * s) : u32x4{0u, 0u, 0u, 0u});
  }
  const int nk = (int)(g.hi - g.lo);
  const uint16_t* kbase = reinterpret_cast<const uint16_t*>(a.k) + (hrow + g.lo) * kDim;
  const uint16_t* vbase = reinterpret_cast<const uint16_t*>(a.v) + (hrow + g.lo) * kDim;
  unsigned char* sK = smem;                          // buffer b: K tile at sK + b * 2 * kKeyTile * KL::kRow
  unsigned char* sV = smem + kKeyTile * KL::kRow;    //           V tile right after it
  const float ls = a.logit_scale;
  auto issue = [&](int k0, int buf) {
    const int bytes = (nk - k0) * 256;
    const i32x4 kr = rsrc_words(kbase + (int64_t)k0 * kDim, bytes);
    const i32x4 vr = rsrc_words(vbase + (int64_t)k0 * kDim, bytes);
    dma_tile<KL, kKeyTile, kQW>(kr, lds_addr(sK + buf * 2 * kKeyTile * KL::kRow), wave, lane);
    dma_tile<KL, kKeyTile, kQW>(vr, lds_addr(sV + buf * 2 * kKeyTile * KL::kRow), wave, lane);
  };
  __syncthreads();   // the linear part's slabs are no longer read
  issue(0, 0);
  int buf = 0;
#pragma unroll 1
  for (int k0 = 0; k0 < nk; k0 += kKeyTile) {
    wait_vmem_all();
    __syncthreads();   // this tile landed everywhere; the other buffer is free
    if (k0 + kKeyTile < nk) issue(k0 + kKeyTile, buf ^ 1);
    const unsigned char* bK = sK + buf * 2 * kKeyTile * KL::kRow;
    const unsigned char* bV = sV + buf * 2 * kKeyTile * KL::kRow;
    buf ^= 1;
    if (!active) continue;
    // both 32-key blocks of the tile: their S and dP MFMAs first, then each block's ds and
    // dq MFMAs (keys past nk have zero K and V rows and are masked out of ds)
    f32x16 St[kKeyTile / 32], Pt[kKeyTile / 32];
#pragma unroll
    for (int kb = 0; kb < kKeyTile / 32; ++kb) {
      bf16x8 kf[8], vf[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        kf[s] = as_bf16x8(lds_read16(bK, KL::a_off(lane, s) + kb * 32 * KL::kRow));
        vf[s] = as_bf16x8(lds_read16(bV, KL::a_off(lane, s) + kb * 32 * KL::kRow));
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) St[kb][i] = Pt[kb][i] = 0.0f;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        St[kb] = mfma32(kf[s], Qf[s], St[kb]);
        Pt[kb] = mfma32(vf[s], DYf[s], Pt[kb]);
      }
    }
#pragma unroll
    for (int kb = 0; kb < kKeyTile / 32; ++kb) {
      bf16x8 kt[4][2];
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const unsigned char* t = bK + (32 * kb + 16 * j) * KL::kRow;
          kt[db][j] = frag_tr_at(t + KL::t_off(lane, db, 0), t + KL::t_off(lane, db, 1));
        }
      // ds of the block; keys past nk (only in the window's last tile) are masked out
      bf16x8 dsb[2];
      auto ds_block = [&](auto masked) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          u32x4 pk;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float d2[2];
#pragma unroll
            for (int q2 = 0; q2 < 2; ++q2) {
              const int i = 8 * j + 2 * e + q2;
              float p = fast_exp2(St[kb][i] * ls - lse_l);
              if (decltype(masked)::value && k0 + 32 * kb + cidx(i, lane) >= nk) p = 0.0f;
              d2[q2] = p * fmaf(Pt[kb][i], us, -dd_l);
            }
            pk[e] = pack_bf16_u32(d2[0], d2[1]);
          }
          dsb[j] = as_bf16x8(pk);
        }
      };
      if (F <= 128 && k0 + kKeyTile <= nk)   // (F = 256: one path, fewer registers)
        ds_block(std::false_type{});
      else
        ds_block(std::true_type{});
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int j = 0; j < 2; ++j) dQ[db] = mfma32(kt[db][j], dsb[j], dQ[db]);
    }
  }
  if (ok) {
    float* out = a.dx + (hrow + row) * kDim;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        const int d = 32 * db + 8 * gi + 4 * (lane >> 5);
        *reinterpret_cast<f32x4*>(out + d) =
            f32x4{dQ[db][4 * gi], dQ[db][4 * gi + 1], dQ[db][4 * gi + 2], dQ[db][4 * gi + 3]};
      }
  }
}

// ---- dk, dv: one workgroup of 8 waves per 128 keys of a chunk, lane = key ----------------
//
// Window part: for every chunk whose window holds the keys (the keys' own chunk and the
// next ones whose overlap reaches back to them), per 32-query block: S = Q K^T and
// dP = dY V^T (rows of Q and dY in kappa order, so the results are B operands over
// queries), p and ds, dv^T += dY^T p, dk^T += Q^T ds (transposing LDS reads). Linear part,
// per key frame present in the tile: U^T = W^T K^T, (G v)^T, phi(k), dphi(k) = G v - h,
// gk = dphi (1 + u) / sqrt(D), dv^T += G^T phi(k)^T, dk^T += W gk^T, for the lanes whose key
// lies in that frame.
// The workgroup's 128 keys of K and V stay in LDS (rows of 256 B padded to 272, read as
// B-operand pieces each block) rather than in registers, which lets two waves share a
// SIMD: waves w and w + 4 take the same 32 keys; 64-query tiles (Q, dY, lse and dy.y by
// direct-to-LDS loads) are double-buffered and wave w takes the first 32-query block of
// each, wave w + 4 the second; in the linear part they take alternate 32-feature blocks.
// Each holds partial dk and dv sums, added through LDS at the end (wave w finishes dk,
// wave w + 4 dv).
constexpr int kKW = 8;
using QL = Swz256;                                        // layout of the Q and dY tiles
constexpr int kQTile = 64;
constexpr int kQBuf = 2 * kQTile * QL::kRow + 2 * kQTile * 4;   // Q, dY rows; lse, dy.y
constexpr int kKV = 2 * 128 * kRowB;                               // K, V of the 128 keys
constexpr int kRed = 2 * 4 * 64 * 64 * 4;                          // partial dk, dv exchange
constexpr int kDkWin = 2 * kQBuf + kKV;
constexpr int kDkLin = kLinLds > kRed ? kLinLds : kRed;
constexpr int kDkLds = kDkWin > kDkLin ? kDkWin : kDkLin;

template <int F>
__global__ void __launch_bounds__(64 * kKW)
__attribute__((amdgpu_waves_per_eu(2, 2)))
bwd_dkdv_kernel(BwdArgs a) {
  constexpr int FS = F < 128 ? F : 128;
  constexpr int RW = 2 * FS + 16;
  __shared__ __attribute__((aligned(16))) unsigned char smem[kDkLds];
  __shared__ float hs[F];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = wave & 3;                               // key group (32 keys)
  const int half = wave >> 2;                            // 0: first block of a tile, 1: second
  int kt;
  const BwdGeo g = bwd_geo(a, blockIdx.x, kt);
  const int kw0 = kt * 128 + kg * 32;                    // first key of the group in the chunk
  const bool active = kw0 < g.rows;
  const int kl = kw0 + (lane & 31);
  const bool ok = active && kl < g.rows;
  const int64_t key = g.row0 + (ok ? kl : 0);            // this lane's key row
  const int64_t hrow = (int64_t)g.bh * a.N;
  unsigned char* sK = smem + 2 * kQBuf;                 // K rows of the 128 keys (272 B)
  unsigned char* sV = sK + 128 * kRowB;
  {
    // K, V rows of the tile's keys (zero past the chunk)
    const int nkeys = g.rows - kt * 128 < 128 ? g.rows - kt * 128 : 128;
    const uint16_t* kb = reinterpret_cast<const uint16_t*>(a.k) + (hrow + g.row0 + kt * 128) * kDim;
    const uint16_t* vb = reinterpret_cast<const uint16_t*>(a.v) + (hrow + g.row0 + kt * 128) * kDim;
    for (int u = tid; u < 128 * 16; u += 64 * kKW) {
      const int r = u >> 4, c = u & 15;
      const bool in = r < nkeys;
      const u32x4 kx = in ? *reinterpret_cast<const u32x4*>(kb + r * kDim + 8 * c) : u32x4{0u, 0u, 0u, 0u};
      const u32x4 vx = in ? *reinterpret_cast<const u32x4*>(vb + r * kDim + 8 * c) : u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(sK + r * kRowB + 16 * c) = kx;
      *reinterpret_cast<u32x4*>(sV + r * kRowB + 16 * c) = vx;
    }
  }
  // this lane's B-operand pieces: key row 32 kg + l mod 32, chunk 2 s + l / 32
  const int kvoff = (32 * kg + (lane & 31)) * kRowB + 16 * (lane >> 5);
  f32x16 dK[4], dV[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dK[db][i] = dV[db][i] = 0.0f;
  const float ls = a.logit_scale, us = a.u_scale;
  const int ab = kappa(lane & 31) * kRowB + 16 * (lane >> 5);
  const int64_t Np = (int64_t)a.Tc * a.HW;
  const int64_t tile_end = g.row0 + (kt * 128 + 128 < g.rows ? kt * 128 + 128 : g.rows);

  // ---- window part ----
  auto chunk_lo = [&](int tq) {
    const int64_t r = tq * Np - (int64_t)a.To * a.HW;
    return r > 0 ? r : (int64_t)0;
  };
  auto chunk_rows = [&](int tq) {
    const int64_t r0 = tq * Np;
    return (int)((r0 + Np < a.N) ? Np : a.N - r0);
  };
  auto issue = [&](int tq, int q0, int b) {
    const int64_t r0 = tq * Np + q0;
    const int bytes = (chunk_rows(tq) - q0) * 256;
    const unsigned base = lds_addr(smem + b * kQBuf);
    const i32x4 qr = rsrc_words(reinterpret_cast<const uint16_t*>(a.q) + (hrow + r0) * kDim, bytes);
    const i32x4 yr = rsrc_words(a.dyb + (hrow + r0) * kDim, bytes);
    dma_tile<QL, kQTile, kKW>(qr, base, wave, lane);
    dma_tile<QL, kQTile, kKW>(yr, base + kQTile * QL::kRow, wave, lane);
    if (wave == 0) {
      const unsigned st = base + 2 * kQTile * QL::kRow;
      dma4(rsrc_words(a.lse + hrow + r0, bytes / 64), st, lane * 4);
      dma4(rsrc_words(a.dvec + hrow + r0, bytes / 64), st + kQTile * 4, lane * 4);
    }
  };
  int tq = g.t, q0 = 0, qbuf = 0;
  bool have = tq < a.n_chunks && chunk_lo(tq) < tile_end;
  if (have) issue(tq, q0, 0);
#pragma unroll 1
  while (have) {
    int ntq = tq, nq0 = q0 + kQTile;
    if (nq0 >= chunk_rows(tq)) {
      ntq = tq + 1;
      nq0 = 0;
    }
    const bool nhave = ntq < a.n_chunks && chunk_lo(ntq) < tile_end;
    wait_vmem_all();
    __syncthreads();   // tile landed everywhere (and K, V staged); the other buffer is free
    if (nhave) issue(ntq, nq0, qbuf ^ 1);
    const unsigned char* sQ = smem + qbuf * kQBuf;
    const unsigned char* sY = sQ + kQTile * QL::kRow;
    const float* sL = reinterpret_cast<const float*>(sQ + 2 * kQTile * QL::kRow);
    const float* sD = sL + kQTile;
    const bool key_in = ok && key >= chunk_lo(tq);
    tq = ntq;
    q0 = nq0;
    have = nhave;
    qbuf ^= 1;
    if (!active) continue;
    const int qb = half;   // this wave's 32-query block of the tile
    f32x16 S, Pd;
#pragma unroll
    for (int i = 0; i < 16; ++i) S[i] = Pd[i] = 0.0f;
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2) {
      const bf16x8 qf = as_bf16x8(lds_read16(sQ, QL::a_off(lane, s2) + qb * 32 * QL::kRow));
      const bf16x8 yf = as_bf16x8(lds_read16(sY, QL::a_off(lane, s2) + qb * 32 * QL::kRow));
      const bf16x8 kf = as_bf16x8(lds_read16(sK, kvoff + 32 * s2));
      const bf16x8 vf = as_bf16x8(lds_read16(sV, kvoff + 32 * s2));
      S = mfma32(qf, kf, S);
      Pd = mfma32(yf, vf, Pd);
    }
    f32x4 Lq[4], Dq[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int qi = 32 * qb + 16 * (r >> 1) + 8 * (lane >> 5) + 4 * (r & 1);
      Lq[r] = *reinterpret_cast<const f32x4*>(sL + qi);
      Dq[r] = *reinterpret_cast<const f32x4*>(sD + qi);
    }
    bf16x8 pb[2], dsb[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      u32x4 pp, pd;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float p2[2], d2[2];
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) {
          const int i = 8 * j + 2 * e + q2;
          const float Lv = Lq[2 * j + (2 * e + q2) / 4][(2 * e + q2) % 4];
          const float Dv = Dq[2 * j + (2 * e + q2) / 4][(2 * e + q2) % 4];
          const float p = key_in ? fast_exp2(S[i] * ls - Lv) : 0.0f;
          p2[q2] = p;
          d2[q2] = p * fmaf(Pd[i], us, -Dv);
        }
        pp[e] = pack_bf16_u32(p2[0], p2[1]);
        pd[e] = pack_bf16_u32(d2[0], d2[1]);
      }
      pb[j] = as_bf16x8(pp);
      dsb[j] = as_bf16x8(pd);
    }
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int o = (32 * qb + 16 * j) * QL::kRow;
        const bf16x8 yt = frag_tr_at(sY + o + QL::t_off(lane, db, 0), sY + o + QL::t_off(lane, db, 1));
        const bf16x8 qt = frag_tr_at(sQ + o + QL::t_off(lane, db, 0), sQ + o + QL::t_off(lane, db, 1));
        dV[db] = mfma32(yt, pb[j], dV[db]);
        dK[db] = mfma32(qt, dsb[j], dK[db]);
      }
  }
  __syncthreads();   // every wave done with the tiles; K, V still in LDS

  // ---- linear part: per key frame of the tile, alternate feature blocks per wave pair ----
  bf16x8 Kf[8], Vf[8];
#pragma unroll
  for (int s2 = 0; s2 < 8; ++s2) {
    Kf[s2] = as_bf16x8(lds_read16(sK, kvoff + 32 * s2));
    Vf[s2] = as_bf16x8(lds_read16(sV, kvoff + 32 * s2));
  }
  const int h = g.bh % a.H;
  const uint16_t* wt = a.wt + (a.w_per_head ? (int64_t)h * F * kDim : 0);
  const uint16_t* w = a.w + (a.w_per_head ? (int64_t)h * kDim * F : 0);
  unsigned char* sWt = smem;
  unsigned char* sG = smem + 128 * kRowB;
  unsigned char* sW = smem + 2 * 128 * kRowB;
  uint16_t* go = a.g_out + (hrow + key) * F;
  const int fr0 = (int)((g.row0 + kt * 128) / a.HW);
  const int fr1 = (int)((tile_end - 1) / a.HW);
  const int my_fr = (int)(key / a.HW);
#pragma unroll 1
  for (int fr = fr0; fr <= fr1; ++fr) {
    const bool mine = ok && my_fr == fr;
    const uint16_t* gimg = a.st_img + ((int64_t)g.bh * a.nslot + fr) * F * kDim;
    const float* hsrc = a.st + ((int64_t)g.bh * a.nslot + fr) * ((int64_t)F * kDim + F) + F * kDim;
#pragma unroll 1
    for (int f0 = 0; f0 < F; f0 += FS) {
      __syncthreads();   // (first pass: K, V read into registers) the slabs are free
      stage_rows(sWt, kRowB, wt + (int64_t)f0 * kDim, kDim, 0, FS, kDim, tid, 64 * kKW);
      stage_rows(sG, kRowB, gimg + (int64_t)f0 * kDim, kDim, 0, FS, kDim, tid, 64 * kKW);
      stage_rows(sW, RW, w, F, f0, kDim, FS, tid, 64 * kKW);
      for (int f = tid; f < FS; f += 64 * kKW) hs[f] = hsrc[f0 + f];
      __syncthreads();
      if (!active) continue;
#pragma unroll 1
      for (int fb = half; fb < FS / 32; fb += 2) {
        f32x16 U, DP;
#pragma unroll
        for (int i = 0; i < 16; ++i) U[i] = DP[i] = 0.0f;
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2) {
          U = mfma32(as_bf16x8(lds_read16(sWt, ab + fb * 32 * kRowB + 32 * s2)), Kf[s2], U);
          DP = mfma32(as_bf16x8(lds_read16(sG, ab + fb * 32 * kRowB + 32 * s2)), Vf[s2], DP);
        }
        bf16x8 psb[2], gkb[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          u32x4 pp, pg;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float ps2[2], gk2[2];
#pragma unroll
            for (int q2 = 0; q2 < 2; ++q2) {
              const int i = 8 * j + 2 * e + q2;
              const int fl = 32 * fb + cidx(i, lane);
              const float u = U[i] * us;
              ps2[q2] = mine ? 1.0f + u + 0.5f * u * u : 0.0f;
              gk2[q2] = mine ? (DP[i] - hs[fl]) * (1.0f + u) * us : 0.0f;
            }
            pp[e] = pack_bf16_u32(ps2[0], ps2[1]);
            pg[e] = pack_bf16_u32(gk2[0], gk2[1]);
          }
          psb[j] = as_bf16x8(pp);
          gkb[j] = as_bf16x8(pg);
          if (mine)
            *reinterpret_cast<u32x4*>(go + f0 + 32 * fb + 16 * j + 8 * (lane >> 5)) = pg;
        }
        const int wb = (lane & 31) * RW + 2 * (32 * fb + 8 * (lane >> 5));
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            dV[db] = mfma32(frag_tr(sG, kRowB, 32 * fb + 16 * j, 32 * db, lane), psb[j], dV[db]);
            dK[db] = mfma32(as_bf16x8(lds_read16(sW, wb + db * 32 * RW + 32 * j)), gkb[j], dK[db]);
          }
      }
    }
  }

  // ---- the two partial sums of each key group: wave w finishes dk, wave w + 4 dv ----
  __syncthreads();   // slabs no longer read
  float* xk = reinterpret_cast<float*>(smem) + kg * 64 * 64;            // dk of wave kg + 4
  float* xv = reinterpret_cast<float*>(smem) + (4 + kg) * 64 * 64;      // dv of wave kg
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      float* dst = (half ? xk : xv) + ((db * 4 + q4) * 64 + lane) * 4;
      const f32x16& src = half ? dK[db] : dV[db];
      *reinterpret_cast<f32x4*>(dst) =
          f32x4{src[4 * q4], src[4 * q4 + 1], src[4 * q4 + 2], src[4 * q4 + 3]};
    }
  __syncthreads();
  f32x16 (&mine4)[4] = half ? dV : dK;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const f32x4 o = *reinterpret_cast<const f32x4*>((half ? xv : xk) + ((db * 4 + q4) * 64 + lane) * 4);
#pragma unroll
      for (int c = 0; c < 4; ++c) mine4[db][4 * q4 + c] += o[c];
    }
  if (ok) {
    float* out = (half ? a.dv : a.dx) + (hrow + key) * kDim;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        const int d = 32 * db + 8 * gi + 4 * (lane >> 5);
        *reinterpret_cast<f32x4*>(out + d) = f32x4{mine4[db][4 * gi], mine4[db][4 * gi + 1],
                                                   mine4[db][4 * gi + 2], mine4[db][4 * gi + 3]};
      }
  }
}

}  // namespace

hipError_t launch_bwd_prep(const void* y, const void* dy, int y_f32, const float* lse, int64_t rows,
                           float us, uint16_t* dyb, uint16_t* gb, float* cvec, float* dvec,
                           hipStream_t stream) {
  dim3 grid((unsigned)((rows + 15) / 16)), block(256);
  hipLaunchKernelGGL(bwd_prep_kernel, grid, block, 0, stream, y, dy, y_f32, lse, rows, us, dyb, gb,
                     cvec, dvec);
  return hipGetLastError();
}

hipError_t launch_state_rows_bf16(const float* S, int64_t s_bh, int64_t s_t, int nst, int BH, int F,
                                  uint16_t* img, hipStream_t stream) {
  dim3 grid((F * kDim / 8 + 255) / 256, nst, BH), block(256);
  hipLaunchKernelGGL(state_rows_bf16_kernel, grid, block, 0, stream, S, s_bh, s_t, nst, F, img);
  return hipGetLastError();
}

hipError_t launch_transpose_w(const void* W, int F, int nW, uint16_t* Wt, hipStream_t stream) {
  dim3 grid((F * kDim + 255) / 256, nW), block(256);
  hipLaunchKernelGGL(transpose_w_kernel, grid, block, 0, stream, (const uint16_t*)W, F, Wt);
  return hipGetLastError();
}

hipError_t launch_suffix_states(const float* part, float* out, int F, int D, int T, int Tc, int To,
                                int BH, hipStream_t stream) {
  const int E = F * D + F;
  dim3 grid((E + 255) / 256, BH), block(256);
  hipLaunchKernelGGL(suffix_states_kernel, grid, block, 0, stream, part, out, E, T, Tc, To);
  return hipGetLastError();
}

hipError_t launch_dw_finalize(const float* parts, int64_t E, int BH, int H, int per_head, int F,
                              float* dW, hipStream_t stream) {
  dim3 grid((kDim * F + 255) / 256, per_head ? H : 1), block(256);
  hipLaunchKernelGGL(dw_finalize_kernel, grid, block, 0, stream, parts, E, BH, H, per_head, F, dW);
  return hipGetLastError();
}

hipError_t launch_bwd_dq(const BwdArgs& a, int F, int nblocks, hipStream_t stream) {
  dim3 grid(nblocks), block(64 * kQW);
  switch (F) {
    case 64:  hipLaunchKernelGGL(bwd_dq_kernel<64>, grid, block, 0, stream, a); break;
    case 128: hipLaunchKernelGGL(bwd_dq_kernel<128>, grid, block, 0, stream, a); break;
    case 256: hipLaunchKernelGGL(bwd_dq_kernel<256>, grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const BwdArgs& a, int F, int nblocks, hipStream_t stream) {
  dim3 grid(nblocks), block(64 * kKW);
  switch (F) {
    case 64:  hipLaunchKernelGGL(bwd_dkdv_kernel<64>, grid, block, 0, stream, a); break;
    case 128: hipLaunchKernelGGL(bwd_dkdv_kernel<128>, grid, block, 0, stream, a); break;
    case 256: hipLaunchKernelGGL(bwd_dkdv_kernel<256>, grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace rehyat
