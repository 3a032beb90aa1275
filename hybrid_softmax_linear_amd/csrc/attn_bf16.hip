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
// column and the sums over keys stay inside the lane pair (l, l^32); the exponentiated
// tile P^T feeds O^T = V^T P^T as the B operand without leaving registers. K tiles
// ([64 keys][128 d]) and V^T tiles ([128 d][64 keys], from a V^T copy in HBM) stream into
// LDS by buffer loads that write LDS directly (no staging registers); rows past the window
// come back as zeros from the buffer descriptor's range check.
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
#include "tiles_bf16.h"

namespace rehyat {

namespace {

constexpr int NW = 4;           // waves per workgroup
constexpr int QW = 64;          // queries per wave
constexpr int QT = NW * QW;     // queries per workgroup
constexpr float kNegBig = -3.0e38f;
constexpr int kStageBytes = kKTileBytes + kVTileBytes;   // 32 KB: K tile + V^T tile
constexpr int kBufRsrcWord3 = 0x00020000;                // gfx9 buffer descriptor word 3

typedef __attribute__((address_space(3))) void lds_void;

struct QRegs {
  bf16x8 op[2][8];              // B operand of S^T = K Q^T: [q block][d step]
};

struct Acc {
  f32x16 O[2][4];               // O^T accumulators: [q block][d block]
  float l[2];                   // partial weight sums of this lane's keys
};

// Per-workgroup geometry of one (head, chunk, query tile).
struct Geo {
  int bh, h, t_local, rows, q_wave0;
  int64_t q_row_base, lo, hi;
  bool has_linear;
};

// Tile sources of one workgroup: K rows of the window and the V^T rows of the window.
struct Src {
  __amdgpu_buffer_rsrc_t k;     // base = first window row, range = nk rows
  __amdgpu_buffer_rsrc_t vt;    // base = V^T of the head (or window), range = its extent
  int vt_ld_bytes;              // bytes between V^T rows (d)
  int vt_key0_bytes;            // byte offset of window key 0 inside a V^T row
  int nk;                       // window length
};

__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0)

// Issue the direct-to-LDS loads of tile kt into one stage (4 + 4 per thread).
__device__ __forceinline__ void tile_dma(const Src& s, int kt, unsigned char* stage, int wave,
                                         int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int it = wave * 4 + i;
    // K: LDS bytes [it*1 KB, +1 KB) hold rows 4it..4it+3; physical chunk lane%16
    const int r = 4 * it + (lane >> 4);
    const int c = (lane & 15) ^ kappa(r & 15);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(s.k, (lds_void*)(stage + it * 1024), 16,
                                             (kt * kTileRows + r) * 256 + c * 16, 0, 0, 0);
    // V^T: LDS bytes [16 KB + it*1 KB, +1 KB) hold d rows 8it..8it+7; physical chunk lane%8
    const int d = 8 * it + (lane >> 3);
    const int kc = (lane & 7) ^ ((d + (d >> 3)) & 7);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        s.vt, (lds_void*)(stage + kKTileBytes + it * 1024), 16,
        d * s.vt_ld_bytes + s.vt_key0_bytes + (kt * kTileRows + 8 * kc) * 2, 0, 0, 0);
  }
}

// S^T block (32 keys x 64 queries) of one 32-key block of the K tile in LDS.
__device__ __forceinline__ void qk_block(f32x16 (&Sc)[2], const unsigned char* kbuf, int kb,
                                         const QRegs& Q, int lane) {
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
}

__device__ __forceinline__ void mask_block(f32x16 (&Sc)[2], int key0, int nk, int lane) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (key0 + cidx(i, lane) >= nk) {
      Sc[0][i] = -__builtin_inff();
      Sc[1][i] = -__builtin_inff();
    }
  }
}

__device__ __forceinline__ float rowmax16(const f32x16& v) {
  float m = fmaxf(fmaxf(v[0], v[1]), v[2]);
#pragma unroll
  for (int i = 3; i < 15; i += 2) m = fmaxf(fmaxf(m, v[i]), v[i + 1]);
  return fmaxf(m, v[15]);
}

// p = 2^(s*ls - m0) as bf16 (the B operand of O^T += V^T P^T); l += sum of the rounded p.
__device__ __forceinline__ void softmax_block(bf16x8 (&P)[2][2], float (&l)[2],
                                              const f32x16 (&Sc)[2], const float (&m0)[2],
                                              float ls) {
  const bf16x2 ones{(bf16)1.0f, (bf16)1.0f};
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      u32x4 pk;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i0 = 8 * j + 2 * e;
        bf16x2 pb = pack_bf16(fast_exp2(Sc[qb][i0] * ls - m0[qb]),
                              fast_exp2(Sc[qb][i0 + 1] * ls - m0[qb]));
        acc = __builtin_amdgcn_fdot2_f32_bf16(pb, ones, acc, false);
        pk[e] = __builtin_bit_cast(unsigned, pb);
      }
      P[qb][j] = as_bf16x8(pk);
    }
    l[qb] += acc;
  }
}

__device__ __forceinline__ void pv_block(Acc& A, const bf16x8 (&P)[2][2], const unsigned char* vbuf,
                                         int kb, int lane) {
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    const int d = 32 * db + (lane & 31);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      bf16x8 av = as_bf16x8(lds_read16(vbuf, vtile_chunk_off(d, 4 * kb + 2 * j + (lane >> 5))));
      A.O[0][db] = mfma32(av, P[0][j], A.O[0][db]);
      A.O[1][db] = mfma32(av, P[1][j], A.O[1][db]);
    }
  }
}

// Linear branch: O = a^L^T = S^T phi(Q)^T (bf16 MFMA) and n^L = phi(q).z per q block
// (full sum over the lane pair). Uses smem as W^T / S^T staging; ends with a barrier.
template <int F>
__device__ __forceinline__ void linear_branch(Acc& A, float (&nlf)[2], const AttnArgs& a,
                                              const Geo& g, const QRegs& Q, unsigned char* smem,
                                              float* zs, int tid, int lane) {
  const uint16_t* W = reinterpret_cast<const uint16_t*>(a.Wq) +
                      (a.w_per_head ? (int64_t)g.h * kDim * F : 0);
  const float* S = a.S + g.bh * a.s_bh + g.t_local * a.s_t;
  const float* z = a.z + g.bh * a.z_bh + g.t_local * a.z_t;
  float nl[2] = {0.0f, 0.0f};
  for (int f = tid; f < F; f += 256) zs[f] = z[f];
  constexpr int FS = F < 128 ? F : 128;   // features per LDS slab
  constexpr int NCH = FS / 8;             // 16-byte chunks per S^T row
  unsigned char* wt = smem;               // [FS][128] bf16, K-tile layout
  unsigned char* st = smem + 32768;       // [128 d][FS] bf16
#pragma unroll 1
  for (int f0 = 0; f0 < F; f0 += FS) {
    if (f0 > 0) __syncthreads();
    stage_wt(wt, W, F, f0, FS, tid);
    // S^T slab: thread reads S[f][4*d4 .. +4] (fp32) and scatters 4 bf16 into column f.
    for (int id = tid; id < FS * 32; id += 256) {
      const int fl = id % FS, d4 = id / FS;
      f32x4 v = *reinterpret_cast<const f32x4*>(S + (int64_t)(f0 + fl) * kDim + 4 * d4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d = 4 * d4 + e;
        *reinterpret_cast<bf16*>(st + d * (FS * 2) + ((((fl >> 3) ^ (d & (NCH - 1)))) << 4) +
                                 ((fl & 7) << 1)) = (bf16)v[e];
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
          A.O[0][db] = mfma32(av, P[0][j], A.O[0][db]);
          A.O[1][db] = mfma32(av, P[1][j], A.O[1][db]);
        }
      }
    }
  }
  nlf[0] = pair_sum(nl[0]);
  nlf[1] = pair_sum(nl[1]);
  __syncthreads();
}

__device__ __forceinline__ void zero_acc(Acc& A) {
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    A.l[qb] = 0.0f;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) A.O[qb][db][i] = 0.0f;
  }
}

// With O = a^L (from linear_branch) and reference m0: O = a^L/n^L * w, l = w (in one lane
// of the pair), w = 2^(log2 n^L - m0), the weight of the linear "key".
__device__ __forceinline__ void scale_linear(Acc& A, const float (&nl)[2], const float (&m0)[2],
                                             int lane) {
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float w = fast_exp2(fast_log2(nl[qb]) - m0[qb]);
    const float sc = w / nl[qb];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) A.O[qb][db][i] *= sc;
    A.l[qb] = (lane < 32) ? w : 0.0f;
  }
}

// One 64-key tile from LDS: per 32-key block, S^T = K Q^T, p = 2^(s*ls - m0), l += sum p,
// O^T += V^T P^T. The last tile of the window masks keys >= nk.
template <bool kLastTile>
__device__ __forceinline__ void process_tile(Acc& A, const float (&m0)[2],
                                             const unsigned char* stage, int kt, int nk,
                                             const QRegs& Q, float ls, int lane) {
  const unsigned char* kbuf = stage;
  const unsigned char* vbuf = stage + kKTileBytes;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int key0 = kt * kTileRows + kb * 32;
    if (kLastTile && key0 >= nk) break;
    f32x16 Sc[2];
    qk_block(Sc, kbuf, kb, Q, lane);
    if (kLastTile) mask_block(Sc, key0, nk, lane);
    bf16x8 P[2][2];
    softmax_block(P, A.l, Sc, m0, ls);
    pv_block(A, P, vbuf, kb, lane);
  }
}

// Row maxima (log2 units) over the 32 keys of block 0 of the tile in stage 0.
__device__ __forceinline__ void peek_block0(float (&mb)[2], const unsigned char* stage, int nk,
                                            const QRegs& Q, float ls, int lane) {
  f32x16 Sc[2];
  qk_block(Sc, stage, 0, Q, lane);
  if (nk < 32) mask_block(Sc, 0, nk, lane);
  mb[0] = pair_max(rowmax16(Sc[0])) * ls;
  mb[1] = pair_max(rowmax16(Sc[1])) * ls;
}

// Exact row maxima over the window (log2 units), for the overflow fallback.
__device__ __forceinline__ void max_sweep(float (&mx)[2], const Src& src, const QRegs& Q,
                                          unsigned char* smem, float ls, int wave, int lane) {
  const int ntiles = (src.nk + kTileRows - 1) / kTileRows;
  mx[0] = mx[1] = kNegBig;
#pragma unroll 1
  for (int kt = 0; kt < ntiles; ++kt) {
    __syncthreads();
    tile_dma(src, kt, smem, wave, lane);
    wait_vmem();
    __syncthreads();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (kt * kTileRows + kb * 32 >= src.nk) break;
      f32x16 Sc[2];
      qk_block(Sc, smem, kb, Q, lane);
      mask_block(Sc, kt * kTileRows + kb * 32, src.nk, lane);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) mx[qb] = fmaxf(mx[qb], rowmax16(Sc[qb]) * ls);
    }
  }
  mx[0] = pair_max(mx[0]);
  mx[1] = pair_max(mx[1]);
  __syncthreads();
}

// The key loop over a window whose tile 0 is already in stage 0: double-buffered
// direct-to-LDS tiles, the last tile peeled (masking).
__device__ __forceinline__ void key_loop(Acc& A, const float (&m0)[2], const Src& src,
                                         const QRegs& Q, unsigned char* smem, float ls, int wave,
                                         int lane) {
  const int nk = src.nk;
  const int ntiles = (nk + kTileRows - 1) / kTileRows;
#pragma unroll 1
  for (int kt = 0; kt < ntiles - 1; ++kt) {
    unsigned char* cur = smem + (kt & 1) * kStageBytes;
    unsigned char* nxt = smem + ((kt & 1) ^ 1) * kStageBytes;
    tile_dma(src, kt + 1, nxt, wave, lane);
    process_tile<false>(A, m0, cur, kt, nk, Q, ls, lane);
    wait_vmem();
    __syncthreads();
  }
  const int kt = ntiles - 1;
  process_tile<true>(A, m0, smem + (kt & 1) * kStageBytes, kt, nk, Q, ls, lane);
  __syncthreads();
}

// Load window tile 0 into stage 0 and fix the reference: m0 = max(mlow, block-0 maxima).
__device__ __forceinline__ void start_window(float (&m0)[2], const float (&mlow)[2],
                                             const Src& src, const QRegs& Q, unsigned char* smem,
                                             float ls, int wave, int lane) {
  tile_dma(src, 0, smem, wave, lane);
  wait_vmem();
  __syncthreads();
  float mb[2];
  peek_block0(mb, smem, src.nk, Q, ls, lane);
  m0[0] = fmaxf(mlow[0], mb[0]);
  m0[1] = fmaxf(mlow[1], mb[1]);
}

template <int F>
__global__ void __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(1, 1)))
hybrid_attn_bf16_kernel(AttnArgs a) {
  // 64 KB: two K/V^T stages during the key loop; W^T and S^T slabs for the linear branch.
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * kStageBytes];
  __shared__ float zs[F];
  __shared__ int bad_flag;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int tile = xcd_remap(blockIdx.x, a.nblocks);

  Geo g;
  g.bh = tile / a.tiles_per_head;
  const int rr = tile - g.bh * a.tiles_per_head;
  g.t_local = rr / a.tiles_per_chunk;
  const int qt = rr - g.t_local * a.tiles_per_chunk;
  const int t = a.chunk0 + g.t_local;
  g.h = g.bh % a.H;
  const int64_t Np = (int64_t)a.Tc * a.HW;
  const int64_t N = (int64_t)a.T * a.HW;
  const int64_t c0 = t * Np;                                  // first token of the chunk
  g.rows = (int)((N - c0) < Np ? (N - c0) : Np);               // query rows of the chunk
  g.lo = (c0 - (int64_t)a.To * a.HW) > 0 ? (c0 - (int64_t)a.To * a.HW) : 0;
  g.hi = c0 + g.rows;
  g.has_linear = a.bidir ? (g.lo > 0 || g.hi < N) : (g.lo > 0);
  g.q_wave0 = qt * QT + wave * QW;
  g.q_row_base = a.step ? 0 : c0;   // row of the chunk start in the q buffer
  if (tid == 0) bad_flag = 0;

  // ---- Q^T operand registers ----------------------------------------------------------
  const uint16_t* qh = reinterpret_cast<const uint16_t*>(a.q) + head_off(g.bh, a.q_rows, kDim);
  QRegs Q;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qrow = g.q_wave0 + qb * 32 + (lane & 31);
    const bool ok = qrow < g.rows;
    const uint16_t* src = qh + (g.q_row_base + (ok ? qrow : 0)) * kDim + 8 * (lane >> 5);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      u32x4 v = ok ? *reinterpret_cast<const u32x4*>(src + 16 * s) : u32x4{0u, 0u, 0u, 0u};
      Q.op[qb][s] = as_bf16x8(v);
    }
  }

  // ---- tile sources: K rows of the window, V^T of the window ---------------------------
  Src src;
  {
    const int nk = (int)(g.hi - g.lo);
    const uint16_t* kbase = reinterpret_cast<const uint16_t*>(a.ka) +
                            head_off(g.bh, a.a_rows, kDim) + (a.step ? 0 : g.lo) * kDim;
    src.k = __builtin_amdgcn_make_buffer_rsrc((void*)kbase, (short)0, nk * 256, kBufRsrcWord3);
    const uint16_t* vbase = reinterpret_cast<const uint16_t*>(a.vt) + g.bh * a.vt_bh +
                            g.t_local * a.vt_t;
    src.vt = __builtin_amdgcn_make_buffer_rsrc((void*)vbase, (short)0, (int)(kDim * a.vt_ld * 2),
                                               kBufRsrcWord3);
    src.vt_ld_bytes = (int)(a.vt_ld * 2);
    src.vt_key0_bytes = (int)((a.vt_key0_is_lo ? g.lo : 0) * 2);
    src.nk = nk;
  }
  const float ls = a.logit_scale;

  // ---- linear branch, then the key loop ------------------------------------------------
  Acc A;
  float m0[2] = {kNegBig, kNegBig}, nl[2] = {1.0f, 1.0f}, ml[2] = {kNegBig, kNegBig};
  zero_acc(A);
  if (g.has_linear) {
    linear_branch<F>(A, nl, a, g, Q, smem, zs, tid, lane);
    ml[0] = fast_log2(nl[0]);
    ml[1] = fast_log2(nl[1]);
  }
  start_window(m0, ml, src, Q, smem, ls, wave, lane);
  if (g.has_linear) scale_linear(A, nl, m0, lane);
  key_loop(A, m0, src, Q, smem, ls, wave, lane);

  // ---- overflow guard: recompute the workgroup with the exact row maxima ---------------
  {
    bool bad = !__builtin_isfinite(A.l[0]) || !__builtin_isfinite(A.l[1]);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) bad |= !__builtin_isfinite(A.O[qb][db][i]);
    if (wave_any(bad) && lane == 0) atomicOr(&bad_flag, 1);
    __syncthreads();
    if (bad_flag) {
      float mx[2];
      max_sweep(mx, src, Q, smem, ls, wave, lane);
      zero_acc(A);
      if (g.has_linear) linear_branch<F>(A, nl, a, g, Q, smem, zs, tid, lane);
      // reference = the exact maximum over the linear weight and every window key: every
      // p <= 1 and l >= 1
      const float mref[2] = {fmaxf(ml[0], mx[0]), fmaxf(ml[1], mx[1])};
      start_window(m0, mref, src, Q, smem, ls, wave, lane);
      if (g.has_linear) scale_linear(A, nl, m0, lane);
      key_loop(A, m0, src, Q, smem, ls, wave, lane);
    }
  }

  // ---- epilogue: y = O / l ------------------------------------------------------------
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qrow = g.q_wave0 + qb * 32 + (lane & 31);
    const float inv = 1.0f / pair_sum(A.l[qb]);
    if (qrow >= g.rows) continue;
    const int64_t off = head_off(g.bh, a.q_rows, kDim) + (g.q_row_base + qrow) * kDim;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        const int d = 32 * db + 8 * gi + 4 * (lane >> 5);
        float v0 = A.O[qb][db][4 * gi + 0] * inv, v1 = A.O[qb][db][4 * gi + 1] * inv;
        float v2 = A.O[qb][db][4 * gi + 2] * inv, v3 = A.O[qb][db][4 * gi + 3] * inv;
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
