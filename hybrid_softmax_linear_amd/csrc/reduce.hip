// reduce.hip - fp32 combination of partial states and the overlap-tail copy.
//
// Partial states are [BH][segments][E] with E = F*D + F (S row-major, then z).
//   fold: S = (init ? 0 : S) + sum of segments (the state update of the chunk-wise RNN,
//         papernotes.org ReHyAt note, key design 4).
// (The scan of the whole-sequence form, which also writes the attention kernel's bf16
// state images, is in state_bf16.hip.)
// Sums run in a fixed order: results are bitwise reproducible.
#include "common.h"

namespace rehyat {

namespace {

__global__ void __launch_bounds__(256)
fold_states_kernel(const float* __restrict__ part, int nseg, float* S, float* z, int F, int D,
                   int init) {
  const int FD = F * D;
  const int E = FD + F;
  const int e = blockIdx.x * 256 + threadIdx.x;
  const int bh = blockIdx.y;
  if (e >= E) return;
  float* dst = (e < FD) ? S + (int64_t)bh * FD + e : z + (int64_t)bh * F + (e - FD);
  float acc = init ? 0.0f : *dst;
  const float* p = part + (int64_t)bh * nseg * E + e;
  for (int s = 0; s < nseg; ++s) acc += p[(int64_t)s * E];
  *dst = acc;
}

__global__ void __launch_bounds__(256)
copy_rows_kernel(const u32x4* __restrict__ sk, const u32x4* __restrict__ sv, u32x4* __restrict__ dk,
                 u32x4* __restrict__ dv, int64_t src_head_units, int64_t src_off_units,
                 int64_t dst_head_units, int64_t units) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int bh = blockIdx.y;
  if (i >= units) return;
  const int64_t s = bh * src_head_units + src_off_units + i;
  const int64_t d = bh * dst_head_units + i;
  dk[d] = sk[s];
  dv[d] = sv[s];
}

__global__ void __launch_bounds__(64) zero_u32_kernel(unsigned* p, int n) {
  for (int i = threadIdx.x; i < n; i += 64) p[i] = 0u;
}

}  // namespace

// Zero n 32-bit words (a fill kernel: callers may capture it in a graph).
hipError_t launch_zero_u32(unsigned* p, int n, hipStream_t stream) {
  hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(64), 0, stream, p, n);
  return hipGetLastError();
}

hipError_t launch_fold_states(const float* part, int nseg, float* S, float* z, int F, int D,
                              int init, int BH, hipStream_t stream) {
  const int E = F * D + F;
  dim3 grid((E + 255) / 256, BH), block(256);
  hipLaunchKernelGGL(fold_states_kernel, grid, block, 0, stream, part, nseg, S, z, F, D, init);
  return hipGetLastError();
}

// Copy `rows` rows of K and V per head (row = row_bytes bytes, a multiple of 16) from row
// src_row0 of the source heads (src_rows rows per head) to rows [0, rows) of the
// destination heads (rows per head = rows).
hipError_t launch_copy_rows(const void* sk, const void* sv, void* dk, void* dv, int64_t src_rows,
                            int64_t src_row0, int64_t rows, int row_bytes, int BH,
                            hipStream_t stream) {
  const int64_t upr = row_bytes / 16;
  const int64_t units = rows * upr;
  if (units == 0) return hipSuccess;
  dim3 grid((unsigned)((units + 255) / 256), BH), block(256);
  hipLaunchKernelGGL(copy_rows_kernel, grid, block, 0, stream, (const u32x4*)sk, (const u32x4*)sv,
                     (u32x4*)dk, (u32x4*)dv, src_rows * upr, src_row0 * upr, units, units);
  return hipGetLastError();
}

}  // namespace rehyat
