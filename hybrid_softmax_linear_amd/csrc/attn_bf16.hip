// attn_bf16.hip - hybrid softmax/linear attention forward on bf16 MFMA (gfx950), D = 128.
//
// One workgroup (4 waves) computes 256 query rows of one chunk of one head:
//   y = (sum_window exp(q.k/sqrt(D)) v + a^L) / (sum_window exp(q.k/sqrt(D)) + n^L)
// (joint normalisation of the softmax and linear branches, papernotes.org ReHyAt note,
// key design 1; window = the chunk plus To earlier frames, key design 2; linear branch
// a^L = phi(q) S, n^L = phi(q) z from the carried state, key design 4).
//
// Each wave owns 64 queries (two 32-query MFMA column blocks). Work is done transposed:
// S^T = K Q^T (A = K from LDS, B = Q^T held in registers), so each lane owns one query
// column and the row max / row sum over keys stay inside the lane pair (l, l^32); the
// exponentiated tile P^T feeds O^T = V^T P^T as the B operand without leaving registers.
//
// The linear branch is folded into the online-softmax state before the key loop: it
// acts as one extra "key" of weight n^L and value a^L/n^L, i.e. the accumulators start
// at O = a^L/n^L, l = 1 with the running max m = log2(n^L). Every later rescale keeps the
// ratio exact, so the result is the unstabilised definition (no stabiliser survives).
// Rescaling is lazy: the running max only moves when a tile exceeds it by more than 2^8,
// so exp2 arguments stay <= 8 and the common path never touches the O accumulators.
#include "tiles_bf16.h"

namespace rehyat {

namespace {

constexpr int NW = 4;           // waves per workgroup
constexpr int QW = 64;          // queries per wave
constexpr int QT = NW * QW;     // queries per workgroup
constexpr float kTau = 8.0f;    // lazy rescale threshold, log2 units
constexpr float kNegBig = -3.0e38f;

struct QRegs {
  bf16x8 op[2][8];              // B operand of S^T = K Q^T: [q block][d step]
};

template <int F>
__global__ void __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(1, 1)))
hybrid_attn_bf16_kernel(AttnArgs a) {
  // 64 KB: two K/V stages during the key loop; W^T and S^T slabs during the prologue.
  __shared__ __attribute__((aligned(16))) unsigned char smem[65536];
  __shared__ float zs[F];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int tile = xcd_remap(blockIdx.x, a.nblocks);
  const int bh = tile / a.tiles_per_head;
  const int rr = tile - bh * a.tiles_per_head;
  const int t_local = rr / a.tiles_per_chunk;
  const int qt = rr - t_local * a.tiles_per_chunk;
  const int t = a.chunk0 + t_local;
  const int h = bh % a.H;

  const int64_t Np = (int64_t)a.Tc * a.HW;
  const int64_t N = (int64_t)a.T * a.HW;
  const int64_t c0 = t * Np;                                // first token of the chunk
  const int rows = (int)((N - c0) < Np ? (N - c0) : Np);     // query rows of the chunk
  const int64_t lo = (c0 - (int64_t)a.To * a.HW) > 0 ? (c0 - (int64_t)a.To * a.HW) : 0;
  const int64_t hi = c0 + rows;
  const bool has_linear = a.bidir ? (lo > 0 || hi < N) : (lo > 0);

  // query rows of this tile, relative to the chunk
  const int q_tile0 = qt * QT;
  const int q_wave0 = q_tile0 + wave * QW;
  const int64_t q_row_base = (a.step ? 0 : c0);   // row of the chunk start in the q buffer

  const uint16_t* qh = reinterpret_cast<const uint16_t*>(a.q) + head_off(bh, a.q_rows, kDim);

  // ---- Q^T operand registers ----------------------------------------------------------
  QRegs Q;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qrow = q_wave0 + qb * 32 + (lane & 31);
    const bool ok = qrow < rows;
    const uint16_t* src = qh + (q_row_base + (ok ? qrow : 0)) * kDim + 8 * (lane >> 5);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      u32x4 v = ok ? *reinterpret_cast<const u32x4*>(src + 16 * s) : u32x4{0u, 0u, 0u, 0u};
      Q.op[qb][s] = as_bf16x8(v);
    }
  }

  f32x16 O[2][4];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) O[qb][db][i] = 0.0f;

  float m[2] = {kNegBig, kNegBig};
  float lsum[2] = {0.0f, 0.0f};

  // ---- prologue: linear branch a^L = phi(q) S_t, n^L = phi(q) z_t -----------------------
  if (has_linear) {
    const uint16_t* W = reinterpret_cast<const uint16_t*>(a.Wq) +
                        (a.w_per_head ? (int64_t)h * kDim * F : 0);
    const float* S = a.S + bh * a.s_bh + t_local * a.s_t;
    const float* z = a.z + bh * a.z_bh + t_local * a.z_t;
    float nl[2] = {0.0f, 0.0f};
    for (int f = tid; f < F; f += 256) zs[f] = z[f];
    constexpr int FS = F < 128 ? F : 128;   // features per LDS slab
    constexpr int NCH = FS / 8;             // 16-byte chunks per S^T row
    unsigned char* wt = smem;               // [FS][128] bf16, K-tile layout
    unsigned char* st = smem + 32768;       // [128 d][FS] bf16
#pragma unroll 1
    for (int f0 = 0; f0 < F; f0 += FS) {
      __syncthreads();
      stage_wt(wt, W, F, f0, FS, tid);
      // S^T slab: thread reads S[f][4*d4 .. +4] (fp32) and scatters 4 bf16 into column f.
      for (int id = tid; id < FS * 32; id += 256) {
        const int fl = id % FS, d4 = id / FS;
        f32x4 v = *reinterpret_cast<const f32x4*>(S + (int64_t)(f0 + fl) * kDim + 4 * d4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int d = 4 * d4 + e;
          bf16 b = (bf16)v[e];
          *reinterpret_cast<bf16*>(st + d * (FS * 2) + ((((fl >> 3) ^ (d & (NCH - 1)))) << 4) +
                                   ((fl & 7) << 1)) = b;
        }
      }
      __syncthreads();
#pragma unroll 1
      for (int fb = 0; fb < FS / 32; ++fb) {
        // U^T block: rows = features 32fb + kappa(l%32) (A = W^T), cols = queries (B = Q^T)
        f32x16 U[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int i = 0; i < 16; ++i) U[qb][i] = 0.0f;
        const int arow = 32 * fb + kappa(lane & 31);
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          bf16x8 av = as_bf16x8(lds_read16(wt, ktile_off(arow, 2 * s + (lane >> 5))));
          U[0] = mfma32(av, Q.op[0][s], U[0]);
          U[1] = mfma32(av, Q.op[1][s], U[1]);
        }
        // phi = 1 + u + u^2/2, rounded to bf16: B operand of a^L^T = S^T phi^T.
        bf16x8 P[2][2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            u32x4 pk;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int i0 = 8 * j + 2 * e;
              float u0 = U[qb][i0] * a.u_scale, u1 = U[qb][i0 + 1] * a.u_scale;
              float p0 = 1.0f + u0 + 0.5f * u0 * u0;
              float p1 = 1.0f + u1 + 0.5f * u1 * u1;
              unsigned w = pack_bf16_u32(p0, p1);
              pk[e] = w;
              const int f = f0 + 32 * fb + cidx(i0, lane);
              nl[qb] += bf16_lo(w) * zs[f] + bf16_hi(w) * zs[f + 1];
            }
            P[qb][j] = as_bf16x8(pk);
          }
        }
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const int d = 32 * db + (lane & 31);
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int c = 4 * fb + 2 * j + (lane >> 5);
            bf16x8 av = as_bf16x8(lds_read16(st, d * (FS * 2) + ((c ^ (d & (NCH - 1))) << 4)));
            O[0][db] = mfma32(av, P[0][j], O[0][db]);
            O[1][db] = mfma32(av, P[1][j], O[1][db]);
          }
        }
      }
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float n_full = pair_sum(nl[qb]);
      const float inv = 1.0f / n_full;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) O[qb][db][i] *= inv;
      m[qb] = fast_log2(n_full);
      lsum[qb] = (lane < 32) ? 1.0f : 0.0f;
    }
    __syncthreads();
  }

  // ---- key loop over the softmax window -----------------------------------------------
  RowSrc ks, vs;
  {
    const int64_t na = a.step ? (c0 - lo) : (hi - lo);
    const int64_t nk = (hi - lo);
    const uint16_t* ka = reinterpret_cast<const uint16_t*>(a.ka) + head_off(bh, a.a_rows, kDim);
    const uint16_t* va = reinterpret_cast<const uint16_t*>(a.va) + head_off(bh, a.a_rows, kDim);
    const uint16_t* kb = reinterpret_cast<const uint16_t*>(a.kb) + head_off(bh, a.b_rows, kDim);
    const uint16_t* vb = reinterpret_cast<const uint16_t*>(a.vb) + head_off(bh, a.b_rows, kDim);
    const int64_t a_row0 = a.step ? (a.a_rows - na) : lo;
    ks = RowSrc{ka, kb, a_row0, na, nk};
    vs = RowSrc{va, vb, a_row0, na, nk};
  }
  const int nk = (int)ks.n;
  const int ntiles = (nk + kTileRows - 1) / kTileRows;
  const float ls = a.logit_scale;

  TileRegs pre;
  tile_load(pre, ks, vs, 0, tid);
  tile_store(pre, smem, smem + kKTileBytes, tid);
  __syncthreads();

#pragma unroll 1
  for (int kt = 0; kt < ntiles; ++kt) {
    const int stage = kt & 1;
    unsigned char* kbuf = smem + stage * (kKTileBytes + kVTileBytes);
    unsigned char* vbuf = kbuf + kKTileBytes;
    const bool more = kt + 1 < ntiles;
    if (more) tile_load(pre, ks, vs, (int64_t)(kt + 1) * kTileRows, tid);

#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key0 = kt * kTileRows + kb * 32;
      if (key0 >= nk) break;
      f32x16 Sc[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int i = 0; i < 16; ++i) Sc[qb][i] = 0.0f;
      const int arow = 32 * kb + kappa(lane & 31);
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        bf16x8 av = as_bf16x8(lds_read16(kbuf, ktile_off(arow, 2 * s + (lane >> 5))));
        Sc[0] = mfma32(av, Q.op[0][s], Sc[0]);
        Sc[1] = mfma32(av, Q.op[1][s], Sc[1]);
      }
      if (key0 + 32 > nk) {   // ragged end of the window: drop keys >= nk
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          if (key0 + cidx(i, lane) >= nk) {
            Sc[0][i] = -__builtin_inff();
            Sc[1][i] = -__builtin_inff();
          }
        }
      }
      bf16x8 P[2][2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        float mx = Sc[qb][0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(mx, Sc[qb][i]);
        if (wave_any(mx * ls > m[qb] + kTau)) {
          const float mnew = fmaxf(m[qb], pair_max(mx) * ls);
          const float alpha = fast_exp2(m[qb] - mnew);
#pragma unroll
          for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) O[qb][db][i] *= alpha;
          lsum[qb] *= alpha;
          m[qb] = mnew;
        }
        const float mm = m[qb];
        float acc = 0.0f;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          u32x4 pk;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i0 = 8 * j + 2 * e;
            float p0 = fast_exp2(Sc[qb][i0] * ls - mm);
            float p1 = fast_exp2(Sc[qb][i0 + 1] * ls - mm);
            bf16x2 pb = pack_bf16(p0, p1);
            acc = __builtin_amdgcn_fdot2_f32_bf16(pb, bf16x2{(bf16)1.0f, (bf16)1.0f}, acc, false);
            pk[e] = __builtin_bit_cast(unsigned, pb);
          }
          P[qb][j] = as_bf16x8(pk);
        }
        lsum[qb] += acc;
      }
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int d = 32 * db + (lane & 31);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          bf16x8 av = as_bf16x8(lds_read16(vbuf, vtile_chunk_off(d, 4 * kb + 2 * j + (lane >> 5))));
          O[0][db] = mfma32(av, P[0][j], O[0][db]);
          O[1][db] = mfma32(av, P[1][j], O[1][db]);
        }
      }
    }

    if (more) {
      unsigned char* nk_buf = smem + (stage ^ 1) * (kKTileBytes + kVTileBytes);
      tile_store(pre, nk_buf, nk_buf + kKTileBytes, tid);
    }
    __syncthreads();
  }

  // ---- epilogue: y = O / l ------------------------------------------------------------
  const int64_t y_row0 = q_row_base;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qrow = q_wave0 + qb * 32 + (lane & 31);
    const float inv = 1.0f / pair_sum(lsum[qb]);
    if (qrow >= rows) continue;
    const int64_t off = head_off(bh, a.q_rows, kDim) + (y_row0 + qrow) * kDim;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * db + 8 * g + 4 * (lane >> 5);
        float v0 = O[qb][db][4 * g + 0] * inv, v1 = O[qb][db][4 * g + 1] * inv;
        float v2 = O[qb][db][4 * g + 2] * inv, v3 = O[qb][db][4 * g + 3] * inv;
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
}

}  // namespace

int attn_bf16_tile_rows() { return QT; }

hipError_t launch_attn_bf16(const AttnArgs& a, int F, hipStream_t stream) {
  dim3 grid(a.nblocks), block(256);
  switch (F) {
    case 64:  hipLaunchKernelGGL(hybrid_attn_bf16_kernel<64>, grid, block, 0, stream, a); break;
    case 128: hipLaunchKernelGGL(hybrid_attn_bf16_kernel<128>, grid, block, 0, stream, a); break;
    case 256: hipLaunchKernelGGL(hybrid_attn_bf16_kernel<256>, grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace rehyat
