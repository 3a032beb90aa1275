// common.h - device types, MFMA operand layouts and launch-argument structs shared by the
// librehyat kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rehyat {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------------------
// v_mfma_f32_32x32x16_bf16 operand layouts (wave64), lane l = 0..63:
//   A (32 x 16): lane l holds row l%32, k = 8*(l/32) .. 8*(l/32)+7
//   B (16 x 32): lane l holds col l%32, k = 8*(l/32) .. 8*(l/32)+7
//   C (32 x 32): lane l, element i holds row 8*(i/4) + 4*(l/32) + (i%4), col l%32
// A C tile has lane = column, so a C tile of X^T (rows = contraction index of the next
// product) can be fed straight back as the B operand of the next MFMA, and as the A
// operand when the lane index is the A row. For that, the rows of the first product are
// loaded in the order kappa(r) (bits 2 and 3 of r swapped): then C element i of lane l
// carries contraction index cidx(i, l) = 16*(i/8) + 8*(l/32) + (i%8), so elements
// 8j..8j+7 are exactly the k-slots of k-step j of a 32x32x16 operand, in natural order.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ int kappa(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}
__device__ __forceinline__ int cidx(int i, int lane) {
  return 16 * (i >> 3) + 8 * (lane >> 5) + (i & 7);
}
// row of C element i of lane l (natural MFMA row, used for the output tiles)
__device__ __forceinline__ int crow(int i, int lane) {
  return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
}

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) {
  return __builtin_bit_cast(bf16x8, v);
}
__device__ __forceinline__ u32x4 as_u32x4(const bf16x8& v) {
  return __builtin_bit_cast(u32x4, v);
}

// Pack two floats into bf16x2 with round-to-nearest-even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16x2 pack_bf16(float a, float b) {
  bf16x2 r;
  r[0] = (bf16)a;
  r[1] = (bf16)b;
  return r;
}
__device__ __forceinline__ unsigned pack_bf16_u32(float a, float b) {
  return __builtin_bit_cast(unsigned, pack_bf16(a, b));
}
__device__ __forceinline__ float bf16_lo(unsigned u) { return __builtin_bit_cast(float, u << 16); }
__device__ __forceinline__ float bf16_hi(unsigned u) { return __builtin_bit_cast(float, u & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(bf16 x) {
  return __builtin_bit_cast(float, ((unsigned)__builtin_bit_cast(unsigned short, x)) << 16);
}

// Reductions over the lane pair (l, l^32) via v_permlane32_swap. With the same value x
// in both operands the instruction returns p0 = {x[l] for l<32, x[l-32] for l>=32} and
// p1 = {x[l+32] for l<32, x[l] for l>=32}: p0 and p1 hold the pair's two values in every
// lane.
__device__ __forceinline__ void pair_vals(float x, float& a, float& b) {
  unsigned u = __builtin_bit_cast(unsigned, x);
  auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  a = __builtin_bit_cast(float, (unsigned)p[0]);
  b = __builtin_bit_cast(float, (unsigned)p[1]);
}
__device__ __forceinline__ float pair_sum(float x) {
  float a, b;
  pair_vals(x, a, b);
  return a + b;
}
__device__ __forceinline__ float pair_max(float x) {
  float a, b;
  pair_vals(x, a, b);
  return fmaxf(a, b);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Wave-uniform "any lane true".
__device__ __forceinline__ bool wave_any(bool p) {
  return __builtin_amdgcn_ballot_w64(p) != 0;
}

// Blocks are handed to the 8 XCDs round-robin (block b runs on XCD b % 8). Remap so that
// consecutive logical tiles (which share K/V windows) land on the same XCD and its L2.
__device__ __forceinline__ int xcd_remap(int b, int nblocks) {
  const int nx = 8;
  int q = nblocks / nx, r = nblocks % nx;
  int x = b % nx, i = b / nx;
  return (x < r) ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
}

// Offsets of a head inside [B, H, rows, cols] tensors use 64-bit arithmetic.
__device__ __forceinline__ int64_t head_off(int bh, int64_t rows, int cols) {
  return (int64_t)bh * rows * cols;
}

// ---------------------------------------------------------------------------------------
// Launch arguments.
// ---------------------------------------------------------------------------------------

// Hybrid attention: one workgroup per (head, chunk, query tile).
// Work queues of the persistent bf16 attention launch: one per XCD of the chip.
constexpr int kAttnQueues = 8;

struct AttnArgs {
  const void* q;        // query rows; head bh starts at q + bh*q_rows*D
  int64_t q_rows;       // rows per head in the q / y buffers
  void* y;              // output, same row layout as q
  // Keys/values of a chunk's softmax window: window row w < na comes from segment A at row
  // (a_row0 + w), otherwise from segment B at row (w - na). Per-head row counts give the
  // head strides. For the whole-sequence form A is the sequence itself and nb = 0.
  const void* ka; const void* va; int64_t a_rows;
  const void* kb; const void* vb; int64_t b_rows;
  // The bf16 attention kernel reads K and V of the window from segment A alone: the whole
  // sequence (window of chunk t at rows [lo, hi)) or, with step set, a gathered window
  // (rows [0, hi - lo)), a_rows rows per head. The single-launch step kernel reads the
  // window's first na = c0 - lo rows from the last na rows of A (the carried tail) and the
  // rest from B (the chunk), as the fp32 kernel does.
  const void* Wq;       // [D, F] or [H, D, F]
  int w_per_head;
  const float* S;       // linear state of (head, chunk): S + bh*s_bh + t*s_t, [F, D]
  const float* z;       //                                 z + bh*z_bh + t*z_t, [F]
  int64_t s_bh, s_t, z_bh, z_t;
  // bf16 path: images of W^T (head h at wt_img + h*wt_img_head bytes) and of S^T (state
  // (bh, t) at st_img + bh*st_img_bh + t*st_img_t bytes) in the LDS slab layout
  const void* wt_img; int64_t wt_img_head;
  const void* st_img; int64_t st_img_bh, st_img_t;
  // bf16 path, feature maps computed ahead (learned / elu maps): phi(q) rows [.][q_rows][F]
  // with the same row indexing as q; NULL: phi(q) = 1 + u + u^2/2 computed in the kernel
  const void* phiq;
  // optional per-row statistic: log2 of the row's joint normaliser n^S + n^L (softmax
  // weights exp(q.k/sqrt(D))), same row indexing as q; NULL: not written
  float* lse;
  int H;
  int HW, Tc, To, T;    // geometry of the whole video
  int n_chunks;         // chunks handled by this launch
  int chunk0;           // index of the first chunk handled (step path: the chunk index)
  int step;             // 1: window = tail (A) + chunk (B); 0: window inside the sequence
  int bidir;
  int y_f32;            // output dtype: 1 fp32, 0 bf16
  int tiles_per_chunk;  // query tiles of a full chunk
  int tiles_last;       // query tiles of the last chunk handled
  int tiles_per_head;
  int nblocks;
  // bf16 path: NULL, one workgroup per query tile; else kAttnQueues per-XCD work counters
  // (zero before the launch) from which a grid of one workgroup per compute unit takes the
  // query tiles
  unsigned* queue;
  float logit_scale;    // log2(e) / sqrt(D)
  float u_scale;        // 1 / sqrt(D)
};

// Backward of the non-recursive form, bf16 path (bwd_bf16.hip). Rows are [BH][N][128]
// unless noted.
struct BwdArgs {
  const void* q; const void* k; const void* v;   // bf16 inputs of the forward
  const uint16_t* dyb;      // dy rounded to bf16
  const uint16_t* gb;       // dy / den rounded to bf16 (den = the row's joint normaliser)
  const float* lse;         // [BH][N] log2(den)
  const float* cvec;        // [BH][N] (dy . y) / den
  const float* dvec;        // [BH][N] (dy . y) / sqrt(D)
  const uint16_t* w;        // the map's W [nW][128][F] (q side in the dq kernel, k side in dkdv)
  const uint16_t* wt;       // its transpose [nW][F][128]
  int w_per_head;
  const uint16_t* st_img;   // bf16 rows [F][128] of per-slot states: + (bh * nslot + slot) * F * 128
  const float* st;          // the fp32 states (F*128 + F floats each), same slots, for z / h
  int nslot;
  float* dx;                // dq (dq kernel) or dk (dkdv kernel), fp32
  float* dv;                // dkdv kernel: dv, fp32
  uint16_t* phi_out;        // dq kernel: phi(q) rows [BH][N][F] bf16
  uint16_t* g_out;          // rows [BH][N][F] bf16 of dphi * (1 + u) / sqrt(D)
  int H, HW, Tc, To, T, N, n_chunks;
  int tiles_per_chunk, tiles_last, tiles_per_head;
  float logit_scale;        // log2(e) / sqrt(D)
  float u_scale;            // 1 / sqrt(D)
};

// Per-segment partial states: one workgroup per (head, segment).
struct StateArgs {
  const void* ka; const void* va; int64_t a_rows; int64_t a_row0;  // rows [0, na) from A
  const void* kb; const void* vb; int64_t b_rows; int64_t b_row0;  // then rows from B
  int64_t na, n;        // rows in A, total rows
  int seg_len;          // rows per segment
  int n_seg;            // segments per head
  const void* Wk; int w_per_head; int H;
  float* part;          // [BH, n_seg, F*D + F] fp32 partial (S then z)
  float u_scale;
  // optional (bf16 path): phi(k) computed ahead, virtual row w of head bh at
  // phik + (bh * phik_rows + w) * F; NULL: phi(k) = 1 + u + u^2/2 from Wk in the kernel
  const void* phik; int64_t phik_rows;
  // optional per-row weights of the z sums (phi rows path only): z += sum_r zw[r] phi(k_r),
  // zw + bh * phik_rows + r; NULL: z += sum_r phi(k_r)
  const float* zw;
};

// Single-launch recurrent step (bf16 path): the grid holds fold_blocks workgroups (one per
// head; the rest of the leading multiple of 8 are idle) ahead of the attention workgroups
// of the chunk. A head's fold workgroup sums the per-frame partials of the window rows no
// later window reaches onto S, z in frame order, into xs, and writes the new tail; the last
// workgroup of the head to finish copies xs into S and z.
struct StepArgs {
  StateArgs fold;       // segments (frames) of the rows folded in (part unused)
  int fold_blocks;      // leading blocks: a multiple of 8, the first BH fold a head
  int per_head;         // workgroups per head that report to counter[bh]
  unsigned* counter;    // [BH]: zero before the launch, left zero by it
  float* xs;            // [BH][F*D + F]: the new S, z of each head
  float* pp;            // [BH][2][F*D + F]: the two frames' partials of a fold round
  float* S; float* z;   // carried state [BH][F][D], [BH][F], updated in place
  int init;             // the state starts empty (first chunk): S = sum of the partials
  const void* kc; const void* vc; int64_t crow;    // the chunk's K, V: crow rows per head
  void* ktail; void* vtail; int64_t trow;          // the new tail's K, V: trow = To*HW rows
};

}  // namespace rehyat
