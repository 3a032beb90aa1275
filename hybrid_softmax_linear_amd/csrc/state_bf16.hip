// state_bf16.hip - linear-branch state on bf16 MFMA (gfx950), D = 128:
//   * per-segment partial sums  dS = phi(K_seg)^T V_seg  (F x D, fp32) and dz = sum phi(K_seg)
//     (the sums s_t, z_t of the chunk-wise RNN, papernotes.org ReHyAt note, key design 4),
//     one segment per workgroup (the tile loads and reductions are in partial_bf16.h);
//   * the feature map phi(x) = 1 + u + u^2/2, u = x W / sqrt(D), as a standalone op.
#include "partial_bf16.h"

namespace rehyat {

namespace {

// Per-segment partials, one segment per workgroup of 4 waves, two workgroups per CU. The
// kernel is bound by HBM latency, so 32-row tiles stream into four LDS stages by
// direct-to-LDS loads (partial_issue: up to three tiles in flight while one is reduced,
// one barrier per tile) and the W^T operand stays in registers. Every tile is reduced by
// partial_tile (partial_bf16.h), with the operand values and MFMA chain order of the
// single-launch step's fold (segment_sums): the two produce the same bits.
constexpr int kPStages = 4;

// two workgroups per CU; F = 256 (two feature blocks per wave) needs the registers of one
constexpr int partial_min_blocks(int F) { return F > 128 ? 1 : 2; }

template <int F>
__global__ void __launch_bounds__(256, partial_min_blocks(F))
state_partial_bf16_kernel(StateArgs a) {
  // four tile stages; W^T is staged in their space first and read into registers
  __shared__ __attribute__((aligned(16))) unsigned char smem[kPStages * kPStage];
  static_assert(F * 256 <= kPStages * kPStage, "W^T staging exceeds the tile stages");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int seg = blockIdx.x % a.n_seg;
  const int bh = blockIdx.x / a.n_seg;
  const uint16_t* W = reinterpret_cast<const uint16_t*>(a.Wk) +
                      (a.w_per_head ? (int64_t)(bh % a.H) * kDim * F : 0);
  stage_wt(smem, W, F, 0, F, tid);
  __syncthreads();
  constexpr int PW = FBlocks<F>::per_wave;
  const bool active = wave < FBlocks<F>::total;
  bf16x8 wf[PW][8];
#pragma unroll
  for (int p = 0; p < PW; ++p) partial_wt_frags(wf[p], smem, wave + 4 * p, lane);
  __syncthreads();   // the stages may now overwrite W^T

  // this segment's rows: wholly in segment A or wholly in segment B (the host's layout)
  const int64_t r0 = (int64_t)seg * a.seg_len;
  const int nrows = segment_rows(a, seg);
  const bool in_a = r0 < a.na;
  const int64_t row0 = in_a ? head_off(bh, a.a_rows, kDim) + (a.a_row0 + r0) * kDim
                            : head_off(bh, a.b_rows, kDim) + (a.b_row0 + r0 - a.na) * kDim;
  const i32x4 kr =
      rsrc_words(reinterpret_cast<const uint16_t*>(in_a ? a.ka : a.kb) + row0, nrows * 256);
  const i32x4 vr =
      rsrc_words(reinterpret_cast<const uint16_t*>(in_a ? a.va : a.vb) + row0, nrows * 256);
  const int ntiles = (nrows + kPRows - 1) / kPRows;
  const unsigned sl = lds_addr(smem);
  const int per_tile = partial_insts<4>(wave);

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
  for (int t = 0; t < kPStages - 1 && t < ntiles; ++t)
    partial_issue<4>(kr, vr, sl + (t % kPStages) * kPStage, t, wave, lane);
#pragma unroll 1
  for (int t = 0; t < ntiles; ++t) {
    // tiles issued after t: up to kPStages - 2 in flight beyond it
    const int later = ntiles - 1 - t;
    wait_vmcnt((later < kPStages - 2 ? later : kPStages - 2) * per_tile);
    __syncthreads();   // tile t landed everywhere; the stage of tile t - 1 is free
    if (t + kPStages - 1 < ntiles)
      partial_issue<4>(kr, vr, sl + ((t + kPStages - 1) % kPStages) * kPStage,
                       t + kPStages - 1, wave, lane);
    if (!active) continue;
    const unsigned char* kt = smem + (t % kPStages) * kPStage;
#pragma unroll
    for (int p = 0; p < PW; ++p)
      partial_tile<4>(kt, kt + kPRegion, wf[p], t * kPRows, nrows, a.u_scale, 0, lane, acc[p],
                      zp[p]);
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
      for (int i = 0; i < 16; ++i) out[(int64_t)(32 * fb + crow(i, lane)) * kDim + d] = acc[p][db][i];
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

// Window gather for the bf16 attention kernel of the streaming step: window rows [0, nk)
// (rows [0, na) from segment A starting at row a_row0, the rest from segment B) -> K and V
// [BH][ld][128], rows >= nk left as they are (the kernel's range check stops at nk). One
// thread per 16-byte chunk, 16 chunks per row.
__global__ void __launch_bounds__(256)
gather_window_bf16_kernel(const uint16_t* ka, const uint16_t* va, int64_t a_rows, int64_t a_row0,
                          const uint16_t* kb, const uint16_t* vb, int64_t b_rows, int64_t na,
                          int64_t nk, uint16_t* k_out, uint16_t* v_out, int64_t ld,
                          int blocks_per_head) {
  const int bh = blockIdx.x / blocks_per_head;
  const int64_t id = (int64_t)(blockIdx.x % blocks_per_head) * 256 + threadIdx.x;
  const int64_t w = id >> 4;
  const int c = (int)(id & 15);
  if (w >= nk) return;
  const int64_t src = (w < na) ? head_off(bh, a_rows, kDim) + (a_row0 + w) * kDim
                               : head_off(bh, b_rows, kDim) + (w - na) * kDim;
  const uint16_t* kp = (w < na) ? ka : kb;
  const uint16_t* vp = (w < na) ? va : vb;
  const int64_t dst = ((int64_t)bh * ld + w) * kDim + 8 * c;
  *reinterpret_cast<u32x4*>(k_out + dst) = *reinterpret_cast<const u32x4*>(kp + src + 8 * c);
  *reinterpret_cast<u32x4*>(v_out + dst) = *reinterpret_cast<const u32x4*>(vp + src + 8 * c);
}

// bf16 images of the linear-branch operands of the attention kernel, laid out byte for
// byte as that kernel's LDS slabs, so it can copy them into LDS with direct loads:
//   S^T image of one state (F x 128 fp32, row f): per slab of FS = min(F, 128) features,
//     128 rows d of FS bf16; feature chunk c (8 features) of row d sits at chunk
//     c ^ (d mod FS/8).
//   W^T image of one W (128 x F bf16, row d): F rows f of 128 bf16; d chunk c of row f
//     sits at chunk c ^ kappa(f mod 16).
// st_image: one block transposes S[f0 .. f0+32)[0 .. 128) of state (t, bh) through LDS.
__device__ __forceinline__ void st_image_block(const float* __restrict__ S, int64_t s_bh,
                                               int64_t s_t, int F, unsigned char* __restrict__ img,
                                               int64_t img_bh, int64_t img_t, int f0, int t,
                                               int bh, float (*tile)[kDim + 1]) {
  const float* src = S + bh * s_bh + t * s_t + (int64_t)f0 * kDim;
  for (int i = threadIdx.x; i < 32 * kDim; i += 256) tile[i / kDim][i % kDim] = src[i];
  __syncthreads();
  const int FS = F < 128 ? F : 128, NCH = FS / 8;
  const int slab = f0 / FS, fl0 = f0 % FS;
  unsigned char* dst = img + bh * img_bh + t * img_t + (int64_t)slab * kDim * FS * 2;
  for (int i = threadIdx.x; i < kDim * 4; i += 256) {
    const int d = i & (kDim - 1), cc = i >> 7;
    const int c = (fl0 >> 3) + cc;
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = pack_bf16_u32(tile[8 * cc + 2 * e][d], tile[8 * cc + 2 * e + 1][d]);
    *reinterpret_cast<u32x4*>(dst + d * FS * 2 + ((c ^ (d & (NCH - 1))) << 4)) = w;
  }
}

// wt_image: one block writes rows f0 .. f0+32 of the W^T image of head h.
__device__ __forceinline__ void wt_image_block(const uint16_t* __restrict__ W, int F,
                                               unsigned char* __restrict__ img, int f0, int h,
                                               uint16_t (*tile)[34]) {
  const uint16_t* src = W + (int64_t)h * kDim * F;
  for (int i = threadIdx.x; i < kDim * 32; i += 256) {
    const int d = i >> 5, fl = i & 31;
    tile[d][fl] = src[(int64_t)d * F + f0 + fl];
  }
  __syncthreads();
  unsigned char* dst = img + (int64_t)h * F * 256;
  for (int i = threadIdx.x; i < 32 * 16; i += 256) {
    const int c = i & 15, fl = i >> 4, f = f0 + fl;
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = (unsigned)tile[8 * c + 2 * e][fl] | ((unsigned)tile[8 * c + 2 * e + 1][fl] << 16);
    *reinterpret_cast<u32x4*>(dst + f * 256 + ((c ^ kappa(f & 15)) << 4)) = w;
  }
}

// The scan of one element (p: its frame-0 partial, frames E apart; s: its chunk-0 state,
// chunks E apart), as scan_states_kernel's blocks do it.
__device__ __forceinline__ void scan_one(const float* __restrict__ p, float* __restrict__ s,
                                         int64_t E, int T, int Tc, int To, int nch, int bidir) {
  float acc = 0.0f;
  int fr = 0;
  for (int t = 0; t < nch; ++t) {
    const int lof = (t * Tc - To) > 0 ? (t * Tc - To) : 0;
#pragma unroll 4
    for (; fr < lof; ++fr) acc += p[fr * E];
    s[t * E] = acc;
  }
  if (bidir) {
    acc = 0.0f;
    fr = T - 1;
    for (int t = nch - 1; t >= 0; --t) {
      const int hif = ((t + 1) * Tc < T) ? (t + 1) * Tc : T;
#pragma unroll 4
      for (; fr >= hif; --fr) acc += p[fr * E];
      s[t * E] += acc;
    }
  }
}

// Per-chunk states from the frame partials part [BH][T][E] (E = F*D + F: S row-major, then
// z) into states [BH][nch][E], each element summed in frame order (papernotes.org ReHyAt
// note, key designs 1 and 4):
//   causal        S_t = frames [0, lo_t/HW)
//   bidirectional S_t = frames [0, lo_t/HW) + frames [hi_t/HW, T) (the complement of the
//                 window)
// Blocks [0, n_s): (bh, 8 features, 32 d), thread (f, d) sums element f*D + d; with img set
// (D = 128) the block also writes the bf16 S^T image of every state it finishes (8 features
// of 32 rows d: one 16-byte chunk per row, through LDS), the layout of st_image_block.
// Blocks [n_s, n_scan): the z elements, one per thread (kept out of the S blocks so that
// their frame loop has no branch and keeps several frames' loads in flight). Blocks from
// n_scan on are the W^T image blocks and the counter-clearing block of linear_images_kernel
// (n_wt, nz as there).
__global__ void __launch_bounds__(256)
scan_states_kernel(const float* __restrict__ part, float* __restrict__ states, int F, int D, int T,
                   int Tc, int To, int nch, int bidir, int n_s, int n_scan,
                   unsigned char* __restrict__ img,
                   int64_t img_bh, int64_t img_t, const uint16_t* __restrict__ W,
                   unsigned char* __restrict__ wimg, int n_wt, unsigned* __restrict__ zp, int nz) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[kDim][34];
  int b = blockIdx.x;
  if (b >= n_scan) {
    b -= n_scan;
    if (b < n_wt) wt_image_block(W, F, wimg, 32 * (b % (F / 32)), b / (F / 32), tile);
    else for (int i = threadIdx.x; i < nz; i += 256) zp[i] = 0u;
    return;
  }
  const int64_t E = (int64_t)F * D + F;
  if (b >= n_s) {
    // z: one element per thread, no image
    b -= n_s;
    const int nzb = (F + 255) / 256;
    const int bh = b / nzb, f = (b % nzb) * 256 + threadIdx.x;
    if (f >= F) return;
    const float* p = part + (int64_t)bh * T * E + (int64_t)F * D + f;
    float* s = states + (int64_t)bh * nch * E + (int64_t)F * D + f;
    scan_one(p, s, E, T, Tc, To, nch, bidir);
    return;
  }
  float (*st)[32] = reinterpret_cast<float (*)[32]>(&tile[0][0]);   // [8 f][32 d]
  const int ndb = D / 32, nfb = F / 8;
  const int db = b % ndb, fb = (b / ndb) % nfb, bh = b / (ndb * nfb);
  const int fl = threadIdx.x >> 5, dl = threadIdx.x & 31;
  const int f = 8 * fb + fl, d = 32 * db + dl;
  const float* p = part + (int64_t)bh * T * E + (int64_t)f * D + d;
  float* s = states + (int64_t)bh * nch * E + (int64_t)f * D + d;
  // bf16 image of state t's 8 x 32 block
  auto image = [&](int t, float x) {
    st[fl][dl] = x;
    __syncthreads();
    if (threadIdx.x < 32) {
      const int FS = F < 128 ? F : 128, NCH = FS / 8;
      const int f0 = 8 * fb, dd = 32 * db + threadIdx.x;
      const int c = (f0 % FS) >> 3;
      unsigned char* dst = img + bh * img_bh + t * img_t + (int64_t)(f0 / FS) * kDim * FS * 2;
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = pack_bf16_u32(st[2 * e][threadIdx.x], st[2 * e + 1][threadIdx.x]);
      *reinterpret_cast<u32x4*>(dst + dd * FS * 2 + ((c ^ (dd & (NCH - 1))) << 4)) = w;
    }
    __syncthreads();
  };
  float acc = 0.0f;
  int fr = 0;
  for (int t = 0; t < nch; ++t) {
    const int lof = (t * Tc - To) > 0 ? (t * Tc - To) : 0;
#pragma unroll 4
    for (; fr < lof; ++fr) acc += p[fr * E];
    s[t * E] = acc;
    if (img && !bidir) image(t, acc);
  }
  if (bidir) {
    acc = 0.0f;
    fr = T - 1;
    for (int t = nch - 1; t >= 0; --t) {
      const int hif = ((t + 1) * Tc < T) ? (t + 1) * Tc : T;
#pragma unroll 4
      for (; fr >= hif; --fr) acc += p[fr * E];
      const float x = s[t * E] + acc;
      s[t * E] = x;
      if (img) image(t, x);
    }
  }
}

// One launch for both images and, optionally, the clearing of nz words at zp (the work
// counters of the attention launch that follows on the same stream): blocks
// [0, n_st) are S^T image blocks (f block fastest, then state t, then bh), the next n_wt
// W^T image blocks (f block fastest, then h), and one last block clears zp when nz > 0.
__global__ void __launch_bounds__(256)
linear_images_kernel(const float* __restrict__ S, int64_t s_bh, int64_t s_t, int nst, int F,
                     unsigned char* __restrict__ img, int64_t img_bh, int64_t img_t,
                     const uint16_t* __restrict__ W, unsigned char* __restrict__ wimg, int n_st,
                     int n_wt, unsigned* __restrict__ zp, int nz) {
  __shared__ __attribute__((aligned(16))) float tile[32 * (kDim + 1)];
  const int nfb = F / 32;
  int b = blockIdx.x;
  if (b < n_st) {
    const int fb = b % nfb, r = b / nfb;
    st_image_block(S, s_bh, s_t, F, img, img_bh, img_t, 32 * fb, r % nst, r / nst,
                   reinterpret_cast<float (*)[kDim + 1]>(tile));
    return;
  }
  b -= n_st;
  if (b < n_wt) {
    wt_image_block(W, F, wimg, 32 * (b % nfb), b / nfb, reinterpret_cast<uint16_t (*)[34]>(tile));
    return;
  }
  for (int i = threadIdx.x; i < nz; i += 256) zp[i] = 0u;
}

// Per-segment partial states from phi(k) rows computed ahead (feature maps other than
// 1 + u + u^2/2): the phi rows of a 64-row tile are staged row-major (rows of 2F + 64
// bytes) and enter dS = phi(K)^T V as the A operand through transposing LDS reads; V is
// staged transposed as in state_partial_bf16_kernel. dz = sum of phi over the tile's rows.
template <int F>
__global__ void __launch_bounds__(256)
state_partial_phi_bf16_kernel(StateArgs a) {
  constexpr int PLD = F * 2 + 64;
  constexpr int PPR = F / 8;                         // 16-byte pieces per phi row
  constexpr int PIT = kTileRows * PPR / 256;         // phi pieces per thread and tile
  __shared__ __attribute__((aligned(16))) unsigned char pt[kTileRows * PLD];
  __shared__ __attribute__((aligned(16))) unsigned char vt[kVTileBytes];
  __shared__ float zws[kTileRows];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int seg = blockIdx.x % a.n_seg;
  const int bh = blockIdx.x / a.n_seg;
  const int64_t r0 = (int64_t)seg * a.seg_len;
  const int64_t r1 = (r0 + a.seg_len < a.n) ? r0 + a.seg_len : a.n;
  const int nrows = (int)(r1 - r0);
  const uint16_t* ph = reinterpret_cast<const uint16_t*>(a.phik) + ((int64_t)bh * a.phik_rows + r0) * F;
  const float* zw = a.zw ? a.zw + (int64_t)bh * a.phik_rows + r0 : nullptr;

  RowSrc vs;
  {
    const uint16_t* va = reinterpret_cast<const uint16_t*>(a.va) + head_off(bh, a.a_rows, kDim);
    const uint16_t* vb = reinterpret_cast<const uint16_t*>(a.vb) + head_off(bh, a.b_rows, kDim);
    const int64_t na_rel = (a.na - r0) > 0 ? (a.na - r0) : 0;
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
  u32x4 pr[PIT], vr[4];
  auto load = [&](int64_t w0) {
#pragma unroll
    for (int it = 0; it < PIT; ++it) {
      const int id = it * 256 + tid, row = id / PPR, c = id - row * PPR;
      pr[it] = (w0 + row < nrows) ? *reinterpret_cast<const u32x4*>(ph + (w0 + row) * F + 8 * c)
                                  : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int id = it * 256 + tid, row = id >> 4, c = id & 15;
      vr[it] = (w0 + row < nrows) ? *reinterpret_cast<const u32x4*>(row_ptr(vs, w0 + row) + c * 8)
                                  : u32x4{0u, 0u, 0u, 0u};
    }
  };
  load(0);
#pragma unroll 1
  for (int ti = 0; ti < ntiles; ++ti) {
    __syncthreads();   // previous tile fully consumed
#pragma unroll
    for (int it = 0; it < PIT; ++it) {
      const int id = it * 256 + tid, row = id / PPR, c = id - row * PPR;
      *reinterpret_cast<u32x4*>(pt + row * PLD + c * 16) = pr[it];
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int id = it * 256 + tid, row = id >> 4, c = id & 15;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const unsigned w = vr[it][e >> 1];
        *reinterpret_cast<uint16_t*>(vt + vtile_off(c * 8 + e, row)) =
            (e & 1) ? (uint16_t)(w >> 16) : (uint16_t)(w & 0xffffu);
      }
    }
    if (zw && tid < kTileRows)
      zws[tid] = (ti * kTileRows + tid < nrows) ? zw[ti * kTileRows + tid] : 0.0f;
    if (ti + 1 < ntiles) load((int64_t)(ti + 1) * kTileRows);
    __syncthreads();
    if (!active) continue;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (ti * kTileRows + kb * 32 >= nrows) break;
#pragma unroll
      for (int p = 0; p < PW; ++p) {
        const int fb = wave + 4 * p;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const bf16x8 af = frag_tr(pt, PLD, 32 * kb + 16 * j, 32 * fb, lane);
          const u32x4 au = as_u32x4(af);
          if (zw) {
            const int rb = 32 * kb + 16 * j + 8 * (lane >> 5);   // rows of this fragment
#pragma unroll
            for (int e = 0; e < 4; ++e)
              zp[p] += bf16_lo(au[e]) * zws[rb + 2 * e] + bf16_hi(au[e]) * zws[rb + 2 * e + 1];
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) zp[p] += bf16_lo(au[e]) + bf16_hi(au[e]);
          }
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            const int d = 32 * db + (lane & 31);
            const bf16x8 bv = as_bf16x8(lds_read16(vt, vtile_chunk_off(d, 4 * kb + 2 * j + (lane >> 5))));
            acc[p][db] = mfma32(af, bv, acc[p][db]);
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

// ---- feature maps of key design 3, materialised as bf16 rows ------------------------------
//
// 1 + elu(x) (F = D): elementwise.
// Learned polynomial map: psi = relu(x W1 + b1) W2 + b2 (W1 [D][h], W2 [h][F]), split into P
// equal parts, part i (1-based) raised to the power i. Computed transposed, lane = row:
// H^T = W1^T X^T and Psi^T = W2^T H^T on bf16 MFMA (fp32 accumulation); with the A rows
// taken in kappa order, the accumulator of H^T (bias, ReLU, rounded to bf16) is directly the
// B operand of the second product. phi is rounded to bf16 on store.

__global__ void __launch_bounds__(256)
phi_elu_bf16_kernel(const uint16_t* __restrict__ x, uint16_t* __restrict__ out, int64_t units) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // 8 elements per unit
  if (i >= units) return;
  const u32x4 v = reinterpret_cast<const u32x4*>(x)[i];
  u32x4 w;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float a = bf16_lo(v[e]), b = bf16_hi(v[e]);
    w[e] = pack_bf16_u32(a > 0.0f ? 1.0f + a : __expf(a), b > 0.0f ? 1.0f + b : __expf(b));
  }
  reinterpret_cast<u32x4*>(out)[i] = w;
}

// Waves per workgroup and features per W2^T slab of the learned map, so that W1^T, one
// W2^T slab and a 32-row staging buffer per wave fit the 160 KB of LDS, and the registers
// of two slabs' addressing (F = 256) fit one wave per SIMD.
template <int F, int HID> struct MlpShape {
  static constexpr int NW = 4;
  static constexpr int FS = F < (HID > 128 ? 64 : 128) ? F : (HID > 128 ? 64 : 128);
};
constexpr int mlp_threads(int F, int HID) { return 256; }
constexpr int kMlpRow = 2 * kDim + 16;   // bytes per staged row: 128 bf16 + 16 bytes of pad
constexpr int kComputeUnits = 256;       // MI355X: one workgroup of the learned map per CU

template <int F, int HID>
constexpr int mlp_lds_bytes() {
  return HID * (2 * kDim + 16) + MlpShape<F, HID>::FS * (2 * HID + 16) +
         MlpShape<F, HID>::NW * 32 * (kMlpRow + 2 * MlpShape<F, HID>::FS + 16) + 4 * (HID + F);
}

// Rows of W1^T (one hidden unit: 128 d), of W2^T (one feature: HID hidden units) and of the
// per-wave row buffers are padded by 16 bytes: row strides of 4 mod 64 words keep the 16
// lanes of a b128 read on distinct banks, and a lane's operand fragments all sit at
// immediate offsets from one address (rows kappa(l%32) + 32*block, 16-byte chunk
// 2s + l/32). Each wave owns 32-row tiles; x rows come in and phi rows go out through its
// buffer with whole-row (coalesced) global accesses. The grid holds as many workgroups as
// run at once; workgroup g takes the g-th equal share of all heads' tiles, restaging the
// parameters where its share crosses into another head.
template <int F, int HID>
__global__ void __launch_bounds__(mlp_threads(F, HID))
phi_mlp_bf16_kernel(const uint16_t* __restrict__ x, int64_t n, const uint16_t* __restrict__ params,
                    int64_t head_elems, int H, int part_shift, uint16_t* __restrict__ out,
                    int BH) {
  constexpr int NW = MlpShape<F, HID>::NW;
  constexpr int FS = MlpShape<F, HID>::FS;
  constexpr int R1 = kDim * 2 + 16;        // bytes per W1^T row
  constexpr int R2 = HID * 2 + 16;         // bytes per W2^T row
  __shared__ __attribute__((aligned(16))) unsigned char w1t[HID * R1];
  __shared__ __attribute__((aligned(16))) unsigned char w2t[FS * R2];
  constexpr int RO = 2 * FS + 16;          // bytes per row of a phi staging buffer
  __shared__ __attribute__((aligned(16))) unsigned char rbuf[NW * 32 * kMlpRow];
  __shared__ __attribute__((aligned(16))) unsigned char obufs[NW * 32 * RO];
  __shared__ float b1s[HID], b2s[F];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  unsigned char* buf = rbuf + wave * 32 * kMlpRow;
  unsigned char* obuf = obufs + wave * 32 * RO;
  const int a1 = kappa(lane & 31) * R1 + 16 * (lane >> 5);        // W1^T fragment base
  const int a2 = kappa(lane & 31) * R2 + 16 * (lane >> 5);        // W2^T fragment base
  const int ax = (lane & 31) * kMlpRow + 16 * (lane >> 5);        // x fragment / phi chunk base
  const int64_t wtiles = (n + 31) / 32;                           // 32-row tiles per head
  const int64_t T = (int64_t)BH * wtiles;
  const int64_t g0 = T * blockIdx.x / gridDim.x, g1 = T * (blockIdx.x + 1) / gridDim.x;
#pragma unroll 1
  for (int64_t s0 = g0; s0 < g1;) {
    const int bh = (int)(s0 / wtiles);
    const int64_t s1 = g1 < (int64_t)(bh + 1) * wtiles ? g1 : (int64_t)(bh + 1) * wtiles;
    const int64_t tb = (int64_t)bh * wtiles;   // global index of the head's first tile
    const uint16_t* p = params + (head_elems ? (int64_t)(bh % H) * head_elems : 0);
    const uint16_t* W1 = p;
    const uint16_t* b1 = W1 + (int64_t)kDim * HID;
    const uint16_t* W2 = b1 + HID;
    const uint16_t* b2 = W2 + (int64_t)HID * F;
    const uint16_t* xh = x + (int64_t)bh * n * kDim;
    uint16_t* oh = out + (int64_t)bh * n * F;
    __syncthreads();   // the previous head's parameters are no longer read
    for (int id = tid; id < kDim * HID / 8; id += 64 * NW) {     // W1^T
      const int r = id / (HID / 8), c = id - r * (HID / 8);
      const u32x4 w = *reinterpret_cast<const u32x4*>(W1 + (int64_t)r * HID + 8 * c);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        *reinterpret_cast<uint16_t*>(w1t + (8 * c + e) * R1 + 2 * r) =
            (e & 1) ? (uint16_t)(w[e >> 1] >> 16) : (uint16_t)(w[e >> 1] & 0xffffu);
    }
    for (int j = tid; j < HID; j += 64 * NW) b1s[j] = bf16_to_f32(((const bf16*)b1)[j]);
    for (int f = tid; f < F; f += 64 * NW) b2s[f] = bf16_to_f32(((const bf16*)b2)[f]);
    // whole-row loads of tile t: piece u = 64 i + lane is row u/16, 16-byte chunk u%16; the
    // buffer descriptor's range (the head's n rows) turns rows past the end into zeros
    const __amdgpu_buffer_rsrc_t xr =
        __builtin_amdgcn_make_buffer_rsrc((void*)xh, (short)0, (int)(n * kDim * 2), kBufRsrcWord3);
    const __amdgpu_buffer_rsrc_t orr =
        __builtin_amdgcn_make_buffer_rsrc((void*)oh, (short)0, (int)(n * F * 2), kBufRsrcWord3);
    auto load_rows = [&](int64_t t, u32x4* xg) {
      const int base = (int)(t - tb) * 32 * kDim * 2 + 16 * lane;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        xg[i] = __builtin_amdgcn_raw_buffer_load_b128(xr, base + 1024 * i, 0, 0);
    };
#pragma unroll 1
    for (int f0 = 0; f0 < F; f0 += FS) {
      if (f0 > 0) __syncthreads();
      for (int id = tid; id < HID * FS / 8; id += 64 * NW) {     // W2^T slab
        const int r = id / (FS / 8), c = id - r * (FS / 8);
        const u32x4 w = *reinterpret_cast<const u32x4*>(W2 + (int64_t)r * F + f0 + 8 * c);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          *reinterpret_cast<uint16_t*>(w2t + (8 * c + e) * R2 + 2 * r) =
              (e & 1) ? (uint16_t)(w[e >> 1] >> 16) : (uint16_t)(w[e >> 1] & 0xffffu);
      }
      __syncthreads();
      // phi rows of the previous tile leave from obuf one tile later, so that their writes
      // are long done when the wave next waits for its loads (loads and stores share one
      // counter); stores past the head's last row fall outside the descriptor's range
      constexpr int CPR = FS / 8;   // 16-byte chunks per row of the slab
      auto store_rows = [&](int64_t tp) {
#pragma unroll
        for (int i = 0; i < 32 * CPR / 64; ++i) {
          const int u = 64 * i + lane, r = u / CPR, c = u - r * CPR;
          const int off = ((int)(tp - tb) * 32 + r) * F * 2 + f0 * 2 + 16 * c;
          __builtin_amdgcn_raw_buffer_store_b128(
              *reinterpret_cast<const u32x4*>(obuf + r * RO + 16 * c), orr, off, 0, 0);
        }
      };
      u32x4 xg[8];
      load_rows(s0 + wave, xg);
      int64_t tprev = -1;
#pragma unroll 1
      for (int64_t t = s0 + wave; t < s1; t += NW) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int u = 64 * i + lane;
          *reinterpret_cast<u32x4*>(buf + (u >> 4) * kMlpRow + 16 * (u & 15)) = xg[i];
        }
        if (tprev >= 0) store_rows(tprev);
        load_rows(t + NW, xg);   // next tile in flight during this one
        bf16x8 xop[8];
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2) xop[s2] = as_bf16x8(lds_read16(buf, ax + 32 * s2));
        f32x16 Ps[FS / 32];
#pragma unroll
        for (int fb = 0; fb < FS / 32; ++fb)
#pragma unroll
          for (int i = 0; i < 16; ++i) Ps[fb][i] = 0.0f;
        // hidden block jb (32 units): H^T block (bias, ReLU, bf16) feeds every output tile.
        // Software-pipelined: block jb+1's dependent chain of 8 MFMAs is interleaved with
        // block jb's independent output-tile MFMAs.
        constexpr int NJ = HID / 32;
        constexpr int L2 = FS / 32 * 2;   // output-tile MFMAs per hidden block
        auto act = [&](const f32x16& Hc, int jb, bf16x8* hb) {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            u32x4 pk;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int i0 = 8 * j + 2 * e;
              const int u = 32 * jb + cidx(i0, lane);
              pk[e] = pack_bf16_u32(fmaxf(Hc[i0] + b1s[u], 0.0f), fmaxf(Hc[i0 + 1] + b1s[u + 1], 0.0f));
            }
            hb[j] = as_bf16x8(pk);
          }
        };
        f32x16 Hc;
#pragma unroll
        for (int i = 0; i < 16; ++i) Hc[i] = 0.0f;
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2)
          Hc = mfma32(as_bf16x8(lds_read16(w1t, a1 + 32 * s2)), xop[s2], Hc);
#pragma unroll 1
        for (int jb = 0; jb < NJ - 1; ++jb) {
          bf16x8 hb[2];
          act(Hc, jb, hb);
#pragma unroll
          for (int i = 0; i < 16; ++i) Hc[i] = 0.0f;
#pragma unroll
          for (int s2 = 0; s2 < (8 > L2 ? 8 : L2); ++s2) {
            if (s2 < 8)
              Hc = mfma32(as_bf16x8(lds_read16(w1t, a1 + (jb + 1) * 32 * R1 + 32 * s2)), xop[s2 & 7], Hc);
            if (s2 < L2)
              Ps[s2 >> 1] = mfma32(as_bf16x8(lds_read16(w2t, a2 + (s2 >> 1) * 32 * R2 + 64 * jb + 32 * (s2 & 1))),
                                   hb[s2 & 1], Ps[s2 >> 1]);
          }
        }
        {
          bf16x8 hb[2];
          act(Hc, NJ - 1, hb);
#pragma unroll
          for (int s2 = 0; s2 < L2; ++s2)
            Ps[s2 >> 1] = mfma32(as_bf16x8(lds_read16(w2t, a2 + (s2 >> 1) * 32 * R2 + 64 * (NJ - 1) + 32 * (s2 & 1))),
                                 hb[s2 & 1], Ps[s2 >> 1]);
        }
        // phi of the slab's features (bias, the power of the feature's part, bf16) into the
        // buffer, then out as whole rows
#pragma unroll
        for (int fb = 0; fb < FS / 32; ++fb) {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            // 8 consecutive features of one part (parts hold a multiple of 8 features)
            const int fl = 32 * fb + 16 * j + 8 * (lane >> 5);
            float psi[8], v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = psi[e] = Ps[fb][8 * j + e] + b2s[f0 + fl + e];
            for (int k2 = (f0 + fl) >> part_shift; k2 > 0; --k2)   // part i: psi^i
#pragma unroll
              for (int e = 0; e < 8; ++e) v[e] *= psi[e];
            u32x4 pk;
#pragma unroll
            for (int e = 0; e < 4; ++e) pk[e] = pack_bf16_u32(v[2 * e], v[2 * e + 1]);
            *reinterpret_cast<u32x4*>(obuf + (lane & 31) * RO + 2 * fl) = pk;
          }
        }
        tprev = t;
      }
      if (tprev >= 0) store_rows(tprev);
    }
    s0 = s1;
  }
}

}  // namespace

hipError_t launch_gather_window_bf16(const void* ka, const void* va, int64_t a_rows, int64_t a_row0,
                                     const void* kb, const void* vb, int64_t b_rows, int64_t na,
                                     int64_t nk, void* k_out, void* v_out, int64_t ld, int BH,
                                     hipStream_t stream) {
  if (nk <= 0) return hipSuccess;
  const int bph = (int)((nk * 16 + 255) / 256);
  dim3 grid(BH * bph), block(256);
  hipLaunchKernelGGL(gather_window_bf16_kernel, grid, block, 0, stream, (const uint16_t*)ka,
                     (const uint16_t*)va, a_rows, a_row0, (const uint16_t*)kb, (const uint16_t*)vb,
                     b_rows, na, nk, (uint16_t*)k_out, (uint16_t*)v_out, ld, bph);
  return hipGetLastError();
}

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

// S^T images of nst states per head (state (bh, t) at S + bh*s_bh + t*s_t, [F][128] fp32)
// into img + bh*img_bh + t*img_t, and the W^T image of each of nW matrices W ([nW][128][F]
// bf16) into wimg + h*F*256 (wimg may be null to skip it), in one launch; with nz > 0 the
// same launch also clears the nz 32-bit words at zp.
hipError_t launch_linear_images_bf16(const float* S, int64_t s_bh, int64_t s_t, int nst, int BH,
                                     int F, void* img, int64_t img_bh, int64_t img_t,
                                     const void* W, int nW, void* wimg, unsigned* zp, int nz,
                                     hipStream_t stream) {
  if (F % 32 != 0 || nz < 0 || (nz > 0 && !zp)) return hipErrorInvalidValue;
  const int n_st = nst > 0 ? (F / 32) * nst * BH : 0;
  const int n_wt = wimg ? (F / 32) * nW : 0;
  const int nblk = n_st + n_wt + (nz > 0 ? 1 : 0);
  if (nblk == 0) return hipSuccess;
  hipLaunchKernelGGL(linear_images_kernel, dim3(nblk), dim3(256), 0, stream, S, s_bh, s_t, nst,
                     F, (unsigned char*)img, img_bh, img_t, (const uint16_t*)W,
                     (unsigned char*)wimg, n_st, n_wt, zp, nz);
  return hipGetLastError();
}

// The per-chunk states (scan_states_kernel); with img set (bf16, D = 128) also their S^T
// images, and in the same launch the W^T images of wimg (if set) and the clearing of nz
// words at zp.
hipError_t launch_scan_states(const float* part, float* states, int F, int D, int T, int Tc,
                              int To, int nch, int bidir, int BH, void* img, int64_t img_bh,
                              int64_t img_t, const void* W, int nW, void* wimg, unsigned* zp,
                              int nz, hipStream_t stream) {
  if (F % 8 != 0 || D % 32 != 0 || ((img || wimg) && (F % 32 != 0 || D != kDim)) || nz < 0 ||
      (nz > 0 && !zp))
    return hipErrorInvalidValue;
  const int n_s = BH * (F / 8) * (D / 32);
  const int n_scan = n_s + BH * ((F + 255) / 256);
  const int n_wt = wimg ? (F / 32) * nW : 0;
  const int nblk = n_scan + n_wt + (nz > 0 ? 1 : 0);
  hipLaunchKernelGGL(scan_states_kernel, dim3(nblk), dim3(256), 0, stream, part, states, F, D, T,
                     Tc, To, nch, bidir, n_s, n_scan, (unsigned char*)img, img_bh, img_t,
                     (const uint16_t*)W, (unsigned char*)wimg, n_wt, zp, nz);
  return hipGetLastError();
}

// phi rows of a feature map of key design 3 into out [BH][n][F] bf16. kind 1: 1 + elu(x)
// (F = D, params unused); kind 2: the learned polynomial map with the parameter blocks
// [W1 D*hid][b1 hid][W2 hid*F][b2 F] (bf16) at params (+ (bh % H) * block if per head).
hipError_t launch_phi_map_bf16(int kind, const void* x, int64_t n, const void* params,
                               int per_head, int H, int hid, int P, int BH, int F, void* out,
                               hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  if (kind == 1) {
    const int64_t units = (int64_t)BH * n * kDim / 8;
    dim3 grid((unsigned)((units + 255) / 256)), block(256);
    hipLaunchKernelGGL(phi_elu_bf16_kernel, grid, block, 0, stream, (const uint16_t*)x,
                       (uint16_t*)out, units);
    return hipGetLastError();
  }
  if (kind != 2 || P < 1 || F % P || F / P < 8) return hipErrorInvalidValue;
  const int part = F / P;                   // F and P are powers of two: part = 2^shift
  int shift = 0;
  while ((1 << shift) < part) ++shift;
  if ((1 << shift) != part) return hipErrorInvalidValue;
  const int64_t head_elems = per_head ? (int64_t)kDim * hid + hid + (int64_t)hid * F + F : 0;
  // as many workgroups as run at once (1 or 2 per compute unit, by LDS), never more tiles'
  // worth than there are
  const int64_t tiles = (int64_t)BH * ((n + 31) / 32);
  const int64_t wg_max = tiles;
  dim3 block(mlp_threads(F, hid));
  const uint16_t* xx = (const uint16_t*)x;
  const uint16_t* pp = (const uint16_t*)params;
  uint16_t* oo = (uint16_t*)out;
#define REHYAT_MLP(FF, HH)                                                                    \
  static_assert(64 * MlpShape<FF, HH>::NW == mlp_threads(FF, HH), "block size");              \
  if (F == FF && hid == HH) {                                                                 \
    int64_t nwg = (int64_t)kComputeUnits * (mlp_lds_bytes<FF, HH>() <= 80 * 1024 ? 2 : 1);      \
    dim3 grid((unsigned)(nwg < wg_max ? nwg : wg_max));                                         \
    hipLaunchKernelGGL((phi_mlp_bf16_kernel<FF, HH>), grid, block, 0, stream, xx, n, pp,        \
                       head_elems, H, shift, oo, BH);                                         \
    return hipGetLastError();                                                                 \
  }
  REHYAT_MLP(64, 64) REHYAT_MLP(64, 128) REHYAT_MLP(64, 256)
  REHYAT_MLP(128, 64) REHYAT_MLP(128, 128) REHYAT_MLP(128, 256)
  REHYAT_MLP(256, 64) REHYAT_MLP(256, 128) REHYAT_MLP(256, 256)
#undef REHYAT_MLP
  return hipErrorInvalidValue;
}

hipError_t launch_state_partial_phi_bf16(const StateArgs& a, int F, int BH, hipStream_t stream) {
  dim3 grid(BH * a.n_seg), block(256);
  switch (F) {
    case 64:  hipLaunchKernelGGL(state_partial_phi_bf16_kernel<64>, grid, block, 0, stream, a); break;
    case 128: hipLaunchKernelGGL(state_partial_phi_bf16_kernel<128>, grid, block, 0, stream, a); break;
    case 256: hipLaunchKernelGGL(state_partial_phi_bf16_kernel<256>, grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace rehyat
