// f32_path.hip - fp32 kernels (dtype REHYAT_F32): feature map, per-segment partial states
// and hybrid attention, in plain fp32 VALU arithmetic (no MFMA rounding of operands).
//
// Same method as the bf16 path (papernotes.org ReHyAt note, key designs 1, 2 and 4): the
// linear branch phi(q) S, phi(q) z seeds the online-softmax accumulators (O = a^L/n^L,
// l = 1, m = log2 n^L), then the softmax window is streamed in tiles of 32 keys with an
// exactly compensated running max, and y = O / l.
#include "common.h"

namespace rehyat {

namespace {

struct RowSrcF {
  const float* a;
  const float* b;
  int64_t a_row0, na, n;
};

template <int D>
__device__ __forceinline__ const float* rowf(const RowSrcF& s, int64_t w) {
  return (w < s.na) ? s.a + (s.a_row0 + w) * D : s.b + (w - s.na) * D;
}

template <int D>
__global__ void __launch_bounds__(256)
hybrid_attn_f32_kernel(AttnArgs a, int F) {
  constexpr int QTF = 64;         // query rows per workgroup
  constexpr int DS = D / 4;       // d-slice per thread
  constexpr int KTF = 32;         // keys per tile
  extern __shared__ __attribute__((aligned(16))) float sm[];
  float* qs = sm;                 // [64][D] during the prologue; K/V tiles afterwards
  float* ph = sm + QTF * D;       // [64][F]
  float* kt = sm;                 // [32][D]
  float* vt = sm + KTF * D;       // [32][D]

  const int tid = threadIdx.x, r = tid >> 2, p = tid & 3;
  const int tile = xcd_remap(blockIdx.x, a.nblocks);
  const int bh = tile / a.tiles_per_head;
  const int rr = tile - bh * a.tiles_per_head;
  const int t_local = rr / a.tiles_per_chunk;
  const int qt = rr - t_local * a.tiles_per_chunk;
  const int t = a.chunk0 + t_local;
  const int h = bh % a.H;
  const int64_t Np = (int64_t)a.Tc * a.HW, N = (int64_t)a.T * a.HW;
  const int64_t c0 = t * Np;
  const int rows = (int)((N - c0) < Np ? (N - c0) : Np);
  const int64_t lo = (c0 - (int64_t)a.To * a.HW) > 0 ? (c0 - (int64_t)a.To * a.HW) : 0;
  const int64_t hi = c0 + rows;
  const bool has_linear = a.bidir ? (lo > 0 || hi < N) : (lo > 0);
  const int64_t q_row_base = a.step ? 0 : c0;
  const int qrow = qt * QTF + r;
  const bool qok = qrow < rows;

  const float* qh = reinterpret_cast<const float*>(a.q) + head_off(bh, a.q_rows, D);
  for (int i = tid; i < QTF * D; i += 256) {
    const int rq = i / D, d = i % D;
    const int qr = qt * QTF + rq;
    qs[i] = (qr < rows) ? qh[(q_row_base + qr) * D + d] : 0.0f;
  }
  __syncthreads();
  float qreg[DS], O[DS];
#pragma unroll
  for (int j = 0; j < DS; ++j) {
    qreg[j] = qs[r * D + p * DS + j];
    O[j] = 0.0f;
  }
  float m = -3.0e38f, l = 0.0f;

  if (has_linear) {
    const float* W = reinterpret_cast<const float*>(a.Wq) + (a.w_per_head ? (int64_t)h * D * F : 0);
    const float* S = a.S + bh * a.s_bh + t_local * a.s_t;
    const float* z = a.z + bh * a.z_bh + t_local * a.z_t;
    for (int f = p; f < F; f += 4) {
      float u = 0.0f;
      for (int d = 0; d < D; ++d) u = fmaf(qs[r * D + d], W[d * F + f], u);
      u *= a.u_scale;
      ph[r * F + f] = 1.0f + u + 0.5f * u * u;
    }
    __syncthreads();
    float nl = 0.0f;
    for (int f = 0; f < F; ++f) {
      const float pf = ph[r * F + f];
      const float* srow = S + (int64_t)f * D + p * DS;
#pragma unroll
      for (int j = 0; j < DS; ++j) O[j] = fmaf(pf, srow[j], O[j]);
      if ((f & 3) == p) nl = fmaf(pf, z[f], nl);
    }
    nl += __shfl_xor(nl, 1);
    nl += __shfl_xor(nl, 2);
    const float inv = 1.0f / nl;
#pragma unroll
    for (int j = 0; j < DS; ++j) O[j] *= inv;
    m = fast_log2(nl);
    l = 1.0f;
  }
  __syncthreads();

  const int64_t na = a.step ? (c0 - lo) : (hi - lo);
  const int64_t nk = hi - lo;
  RowSrcF ks{reinterpret_cast<const float*>(a.ka) + head_off(bh, a.a_rows, D),
             reinterpret_cast<const float*>(a.kb) + head_off(bh, a.b_rows, D),
             a.step ? (a.a_rows - na) : lo, na, nk};
  RowSrcF vs{reinterpret_cast<const float*>(a.va) + head_off(bh, a.a_rows, D),
             reinterpret_cast<const float*>(a.vb) + head_off(bh, a.b_rows, D),
             ks.a_row0, na, nk};
  const float ls = a.logit_scale;
  for (int64_t k0 = 0; k0 < nk; k0 += KTF) {
    for (int i = tid; i < KTF * D; i += 256) {
      const int kr = i / D, d = i % D;
      const int64_t w = k0 + kr;
      kt[i] = (w < nk) ? rowf<D>(ks, w)[d] : 0.0f;
      vt[i] = (w < nk) ? rowf<D>(vs, w)[d] : 0.0f;
    }
    __syncthreads();
    float s[KTF];
    float mt = -__builtin_inff();
#pragma unroll
    for (int j = 0; j < KTF; ++j) {
      float acc = 0.0f;
#pragma unroll
      for (int e = 0; e < DS; ++e) acc = fmaf(qreg[e], kt[j * D + p * DS + e], acc);
      acc += __shfl_xor(acc, 1);
      acc += __shfl_xor(acc, 2);
      s[j] = (k0 + j < nk) ? acc * ls : -__builtin_inff();
      mt = fmaxf(mt, s[j]);
    }
    const float mnew = fmaxf(m, mt);
    const float alpha = fast_exp2(m - mnew);
    l *= alpha;
#pragma unroll
    for (int e = 0; e < DS; ++e) O[e] *= alpha;
    m = mnew;
#pragma unroll
    for (int j = 0; j < KTF; ++j) {
      const float pj = fast_exp2(s[j] - m);
      l += pj;
#pragma unroll
      for (int e = 0; e < DS; ++e) O[e] = fmaf(pj, vt[j * D + p * DS + e], O[e]);
    }
    __syncthreads();
  }
  if (qok) {
    const float inv = 1.0f / l;
    if (a.lse && p == 0) a.lse[(int64_t)bh * a.q_rows + q_row_base + qrow] = m + fast_log2(l);
    const int64_t off = head_off(bh, a.q_rows, D) + (q_row_base + qrow) * D + p * DS;
#pragma unroll
    for (int e = 0; e < DS; ++e) {
      const float val = O[e] * inv;
      if (a.y_f32) reinterpret_cast<float*>(a.y)[off + e] = val;
      else reinterpret_cast<bf16*>(a.y)[off + e] = (bf16)val;
    }
  }
}

template <int D>
__global__ void __launch_bounds__(256)
state_partial_f32_kernel(StateArgs a, int F) {
  constexpr int RB = 16;          // rows per block
  __shared__ float kt[RB][D];
  __shared__ float vt[RB][D];
  __shared__ float wt[D][16];
  __shared__ float ph[RB][16];
  const int tid = threadIdx.x;
  const int seg = blockIdx.x % a.n_seg, bh = blockIdx.x / a.n_seg, h = bh % a.H;
  const int f0 = blockIdx.y * 16;
  const int fl = tid >> 4, dl = tid & 15;
  const int64_t r0 = (int64_t)seg * a.seg_len;
  const int64_t r1 = (r0 + a.seg_len < a.n) ? r0 + a.seg_len : a.n;
  const float* W = reinterpret_cast<const float*>(a.Wk) + (a.w_per_head ? (int64_t)h * D * F : 0);
  for (int i = tid; i < D * 16; i += 256) wt[i / 16][i % 16] = W[(i / 16) * F + f0 + (i % 16)];
  const float* ka = reinterpret_cast<const float*>(a.ka) + head_off(bh, a.a_rows, D);
  const float* va = reinterpret_cast<const float*>(a.va) + head_off(bh, a.a_rows, D);
  const float* kb = reinterpret_cast<const float*>(a.kb) + head_off(bh, a.b_rows, D);
  const float* vb = reinterpret_cast<const float*>(a.vb) + head_off(bh, a.b_rows, D);
  constexpr int ND = D / 16;
  float acc[ND];
#pragma unroll
  for (int j = 0; j < ND; ++j) acc[j] = 0.0f;
  float zacc = 0.0f;
  for (int64_t rb = r0; rb < r1; rb += RB) {
    __syncthreads();
    for (int i = tid; i < RB * D; i += 256) {
      const int rr = i / D, d = i % D;
      const int64_t g = rb + rr;   // virtual row
      float kv = 0.0f, vv = 0.0f;
      if (g < r1) {
        const float* kp = (g < a.na) ? ka + (a.a_row0 + g) * D : kb + (a.b_row0 + g - a.na) * D;
        const float* vp = (g < a.na) ? va + (a.a_row0 + g) * D : vb + (a.b_row0 + g - a.na) * D;
        kv = kp[d];
        vv = vp[d];
      }
      kt[rr][d] = kv;
      vt[rr][d] = vv;
    }
    __syncthreads();
    {
      const int rr = tid >> 4, ff = tid & 15;
      float u = 0.0f;
      for (int d = 0; d < D; ++d) u = fmaf(kt[rr][d], wt[d][ff], u);
      u *= a.u_scale;
      ph[rr][ff] = (rb + rr < r1) ? 1.0f + u + 0.5f * u * u : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      const float pf = ph[rr][fl];
#pragma unroll
      for (int j = 0; j < ND; ++j) acc[j] = fmaf(pf, vt[rr][dl + 16 * j], acc[j]);
      if (dl == 0) zacc += pf;
    }
  }
  const int E = F * D + F;
  float* out = a.part + ((int64_t)bh * a.n_seg + seg) * E;
#pragma unroll
  for (int j = 0; j < ND; ++j) out[(int64_t)(f0 + fl) * D + dl + 16 * j] = acc[j];
  if (dl == 0) out[F * D + f0 + fl] = zacc;
}

template <int D>
__global__ void __launch_bounds__(256)
phi_f32_kernel(const float* x, int64_t n, const float* Wall, int w_per_head, int H, float* out,
               int F, float u_scale, int tiles_per_head) {
  __shared__ float xs[64][D];
  const int tid = threadIdx.x;
  const int bh = blockIdx.x / tiles_per_head, ti = blockIdx.x % tiles_per_head, h = bh % H;
  const float* W = Wall + (w_per_head ? (int64_t)h * D * F : 0);
  const int64_t row0 = (int64_t)ti * 64;
  const float* xh = x + head_off(bh, n, D);
  for (int i = tid; i < 64 * D; i += 256) {
    const int rr = i / D, d = i % D;
    xs[rr][d] = (row0 + rr < n) ? xh[(row0 + rr) * D + d] : 0.0f;
  }
  __syncthreads();
  for (int i = tid; i < 64 * F; i += 256) {
    const int rr = i / F, f = i % F;
    if (row0 + rr >= n) continue;
    float u = 0.0f;
    for (int d = 0; d < D; ++d) u = fmaf(xs[rr][d], W[d * F + f], u);
    u *= u_scale;
    out[head_off(bh, n, F) + (row0 + rr) * F + f] = 1.0f + u + 0.5f * u * u;
  }
}

}  // namespace

int attn_f32_tile_rows() { return 64; }

hipError_t launch_attn_f32(const AttnArgs& a, int D, int F, hipStream_t stream) {
  dim3 grid(a.nblocks), block(256);
  const size_t lds = (size_t)(64 * D + 64 * F) * sizeof(float);
  if (D == 64) {
    hipError_t e = hipFuncSetAttribute((const void*)hybrid_attn_f32_kernel<64>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(hybrid_attn_f32_kernel<64>, grid, block, lds, stream, a, F);
  } else if (D == 128) {
    hipError_t e = hipFuncSetAttribute((const void*)hybrid_attn_f32_kernel<128>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(hybrid_attn_f32_kernel<128>, grid, block, lds, stream, a, F);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_state_partial_f32(const StateArgs& a, int D, int F, int BH, hipStream_t stream) {
  dim3 grid(BH * a.n_seg, F / 16), block(256);
  if (D == 64) hipLaunchKernelGGL(state_partial_f32_kernel<64>, grid, block, 0, stream, a, F);
  else if (D == 128) hipLaunchKernelGGL(state_partial_f32_kernel<128>, grid, block, 0, stream, a, F);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_phi_f32(const void* x, int64_t n, const void* W, int w_per_head, int H, int BH,
                          int D, int F, void* out, float u_scale, hipStream_t stream) {
  const int tph = (int)((n + 63) / 64);
  dim3 grid(BH * tph), block(256);
  const float* xx = reinterpret_cast<const float*>(x);
  const float* ww = reinterpret_cast<const float*>(W);
  float* oo = reinterpret_cast<float*>(out);
  if (D == 64) hipLaunchKernelGGL(phi_f32_kernel<64>, grid, block, 0, stream, xx, n, ww, w_per_head, H, oo, F, u_scale, tph);
  else if (D == 128) hipLaunchKernelGGL(phi_f32_kernel<128>, grid, block, 0, stream, xx, n, ww, w_per_head, H, oo, F, u_scale, tph);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace rehyat
