// api.cpp - the librehyat C ABI (include/rehyat.h): argument checks, workspace layout and
// kernel orchestration on the caller's stream. Host code only; kernels live in *.hip.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/rehyat.h"
#include "common.h"

namespace rehyat {
hipError_t launch_attn_bf16(const AttnArgs& a, int F, hipStream_t stream);
hipError_t launch_zero_u32(unsigned* p, int n, hipStream_t stream);
bool attn_bf16_persistent(int nblocks);
hipError_t launch_step_bf16(const AttnArgs& a, const StepArgs& s, int F, hipStream_t stream);
int attn_bf16_tile_rows();
hipError_t launch_attn_f32(const AttnArgs& a, int D, int F, hipStream_t stream);
int attn_f32_tile_rows();
hipError_t launch_state_partial_bf16(const StateArgs& a, int F, int BH, hipStream_t stream);
hipError_t launch_state_partial_f32(const StateArgs& a, int D, int F, int BH, hipStream_t stream);
hipError_t launch_phi_bf16(const void* x, int64_t n, const void* W, int w_per_head, int H, int BH,
                           int F, void* out, int out_f32, float u_scale, hipStream_t stream);
hipError_t launch_phi_f32(const void* x, int64_t n, const void* W, int w_per_head, int H, int BH,
                          int D, int F, void* out, float u_scale, hipStream_t stream);
hipError_t launch_scan_states(const float* part, float* states, int F, int D, int T, int Tc,
                              int To, int nch, int bidir, int BH, void* img, int64_t img_bh,
                              int64_t img_t, const void* W, int nW, void* wimg, unsigned* zp,
                              int nz, hipStream_t stream);
hipError_t launch_fold_states(const float* part, int nseg, float* S, float* z, int F, int D,
                              int init, int BH, hipStream_t stream);
hipError_t launch_gather_window_bf16(const void* ka, const void* va, int64_t a_rows, int64_t a_row0,
                                     const void* kb, const void* vb, int64_t b_rows, int64_t na,
                                     int64_t nk, void* k_out, void* v_out, int64_t ld, int BH,
                                     hipStream_t stream);
hipError_t launch_copy_rows(const void* sk, const void* sv, void* dk, void* dv, int64_t src_rows,
                            int64_t src_row0, int64_t rows, int row_bytes, int BH,
                            hipStream_t stream);
hipError_t launch_linear_images_bf16(const float* S, int64_t s_bh, int64_t s_t, int nst, int BH,
                                     int F, void* img, int64_t img_bh, int64_t img_t,
                                     const void* W, int nW, void* wimg, unsigned* zp, int nz,
                                     hipStream_t stream);
hipError_t launch_phi_map_bf16(int kind, const void* x, int64_t n, const void* params,
                               int per_head, int H, int hid, int P, int BH, int F, void* out,
                               hipStream_t stream);
hipError_t launch_state_partial_phi_bf16(const StateArgs& a, int F, int BH, hipStream_t stream);
hipError_t launch_bwd_prep(const void* y, const void* dy, int y_f32, const float* lse, int64_t rows,
                           float us, uint16_t* dyb, uint16_t* gb, float* cvec, float* dvec,
                           hipStream_t stream);
hipError_t launch_state_rows_bf16(const float* S, int64_t s_bh, int64_t s_t, int nst, int BH, int F,
                                  uint16_t* img, hipStream_t stream);
hipError_t launch_transpose_w(const void* W, int F, int nW, uint16_t* Wt, hipStream_t stream);
hipError_t launch_suffix_states(const float* part, float* out, int F, int D, int T, int Tc, int To,
                                int BH, hipStream_t stream);
hipError_t launch_dw_finalize(const float* parts, int64_t E, int BH, int H, int per_head, int F,
                              float* dW, hipStream_t stream);
hipError_t launch_bwd_dq(const BwdArgs& a, int F, int nblocks, hipStream_t stream);
hipError_t launch_bwd_dkdv(const BwdArgs& a, int F, int nblocks, hipStream_t stream);
}  // namespace rehyat

using namespace rehyat;

namespace {

thread_local char g_err[512] = "";

rehyat_status fail(rehyat_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

rehyat_status ok() {
  g_err[0] = '\0';
  return REHYAT_OK;
}

rehyat_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(REHYAT_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t esize(int dtype) { return dtype == REHYAT_BF16 ? 2 : 4; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

constexpr int64_t kMaxElems = (int64_t)1 << 31;

// Checks shared by every entry point.
rehyat_status check_desc(const rehyat_desc* d) {
  if (!d) return fail(REHYAT_ERR_NULL, "desc is NULL");
  if (d->dtype != REHYAT_F32 && d->dtype != REHYAT_BF16)
    return fail(REHYAT_ERR_DTYPE, "dtype %d unknown", d->dtype);
  if (d->y_dtype != REHYAT_F32 && d->y_dtype != REHYAT_BF16)
    return fail(REHYAT_ERR_DTYPE, "y_dtype %d unknown", d->y_dtype);
  if (d->mode != REHYAT_CAUSAL && d->mode != REHYAT_BIDIR)
    return fail(REHYAT_ERR_DTYPE, "mode %d unknown", d->mode);
  if (d->w_per_head != 0 && d->w_per_head != 1)
    return fail(REHYAT_ERR_SHAPE, "w_per_head must be 0 or 1");
  if (d->B < 1 || d->H < 1 || d->T < 1 || d->HW < 1 || d->Tc < 1 || d->To < 0 || d->D < 1 ||
      d->F < 1)
    return fail(REHYAT_ERR_SHAPE, "B, H, T, HW, Tc, D, F must be >= 1 and To >= 0");
  if (d->dtype == REHYAT_BF16) {
    if (d->D != 128) return fail(REHYAT_ERR_UNSUPPORTED, "bf16 path supports D = 128 (got %d)", d->D);
    if (d->F != 64 && d->F != 128 && d->F != 256)
      return fail(REHYAT_ERR_UNSUPPORTED, "bf16 path supports F in {64,128,256} (got %d)", d->F);
  } else {
    if (d->D != 64 && d->D != 128)
      return fail(REHYAT_ERR_UNSUPPORTED, "fp32 path supports D in {64,128} (got %d)", d->D);
    if (d->F % 16 != 0 || d->F > 256)
      return fail(REHYAT_ERR_UNSUPPORTED, "fp32 path supports F = 16..256, multiple of 16 (got %d)", d->F);
  }
  if (d->phi_kind != REHYAT_PHI_POLY2 && d->phi_kind != REHYAT_PHI_ELU &&
      d->phi_kind != REHYAT_PHI_MLP)
    return fail(REHYAT_ERR_DTYPE, "phi_kind %d unknown", d->phi_kind);
  if (d->phi_kind != REHYAT_PHI_POLY2 && d->dtype != REHYAT_BF16)
    return fail(REHYAT_ERR_UNSUPPORTED, "phi_kind %d needs dtype bf16", d->phi_kind);
  if (d->phi_kind == REHYAT_PHI_ELU && d->F != d->D)
    return fail(REHYAT_ERR_SHAPE, "1 + elu needs F = D (got F = %d, D = %d)", d->F, d->D);
  if (d->phi_kind == REHYAT_PHI_MLP) {
    if (d->phi_hidden != 64 && d->phi_hidden != 128 && d->phi_hidden != 256)
      return fail(REHYAT_ERR_UNSUPPORTED, "phi_hidden must be 64, 128 or 256 (got %d)", d->phi_hidden);
    if (d->phi_parts < 1 || d->F % d->phi_parts != 0)
      return fail(REHYAT_ERR_SHAPE, "F = %d does not split into phi_parts = %d parts", d->F, d->phi_parts);
    if (d->F / d->phi_parts < 8)
      return fail(REHYAT_ERR_UNSUPPORTED, "parts of fewer than 8 features (F = %d, phi_parts = %d)",
                  d->F, d->phi_parts);
  }
  const int64_t N = (int64_t)d->T * d->HW;
  const int64_t BH = (int64_t)d->B * d->H;
  const int64_t width = d->D > d->F ? d->D : d->F;
  if (BH * N * width >= kMaxElems) return fail(REHYAT_ERR_SHAPE, "tensor too large (>= 2^31 elements)");
  if ((int64_t)d->Tc * d->HW >= kMaxElems / 256) return fail(REHYAT_ERR_SHAPE, "chunk too large");
  return REHYAT_OK;
}

int n_chunks(const rehyat_desc* d) { return (d->T + d->Tc - 1) / d->Tc; }

// Feature maps of kind 1 and 2 are evaluated ahead into bf16 phi rows.
bool phi_ahead(const rehyat_desc* d) { return d->phi_kind != REHYAT_PHI_POLY2; }
bool needs_w(const rehyat_desc* d) { return d->phi_kind != REHYAT_PHI_ELU; }

// Bytes of one W argument (all heads).
size_t w_bytes(const rehyat_desc* d) {
  const size_t heads = d->w_per_head ? d->H : 1;
  if (d->phi_kind == REHYAT_PHI_ELU) return 0;
  if (d->phi_kind == REHYAT_PHI_MLP) {
    const size_t h = d->phi_hidden;
    return heads * ((size_t)d->D * h + h + h * d->F + d->F) * 2;
  }
  return heads * d->D * d->F * (d->dtype == REHYAT_BF16 ? 2 : 4);
}

// bf16 phi rows of n rows per head.
size_t phi_rows_bytes(const rehyat_desc* d, int64_t n) {
  return (size_t)d->B * d->H * (size_t)n * d->F * 2;
}

hipError_t launch_phi_rows(const rehyat_desc* d, const void* x, int64_t n, const void* W,
                           void* out, hipStream_t s) {
  return launch_phi_map_bf16(d->phi_kind, x, n, W, d->w_per_head, d->H, d->phi_hidden,
                             d->phi_parts, d->B * d->H, d->F, out, s);
}

constexpr size_t kQueueBytes = 256;   // work counters of the persistent attention launch

size_t state_elems(const rehyat_desc* d) { return (size_t)d->F * d->D + d->F; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

// ---- kernel timing ----------------------------------------------------------------------
constexpr int kMaxTimed = 4096;
struct Timing {
  bool enabled = false;
  int which = 1;   // kernel whose launches are timed (rehyat_timing_enable's argument)
  bool created = false;
  int count = 0;
  hipEvent_t ev[2 * kMaxTimed];
};
Timing g_timing;

void timed_begin(hipStream_t s, int which = 1) {
  if (g_timing.enabled && g_timing.which == which && g_timing.count < kMaxTimed)
    (void)hipEventRecord(g_timing.ev[2 * g_timing.count], s);
}
void timed_end(hipStream_t s, int which = 1) {
  if (g_timing.enabled && g_timing.which == which && g_timing.count < kMaxTimed) {
    (void)hipEventRecord(g_timing.ev[2 * g_timing.count + 1], s);
    g_timing.count++;
  }
}

hipError_t launch_attention(const rehyat_desc* d, AttnArgs& a, hipStream_t s) {
  timed_begin(s);
  hipError_t e = (d->dtype == REHYAT_BF16) ? launch_attn_bf16(a, d->F, s)
                                           : launch_attn_f32(a, d->D, d->F, s);
  timed_end(s);
  return e;
}

hipError_t launch_partial(const rehyat_desc* d, const StateArgs& sa, hipStream_t s) {
  const int BH = d->B * d->H;
  if (sa.phik) return launch_state_partial_phi_bf16(sa, d->F, BH, s);
  return (d->dtype == REHYAT_BF16) ? launch_state_partial_bf16(sa, d->F, BH, s)
                                   : launch_state_partial_f32(sa, d->D, d->F, BH, s);
}

void fill_tiles(AttnArgs& a, const rehyat_desc* d, int nch_launch, int last_rows) {
  const int QT = (d->dtype == REHYAT_BF16) ? attn_bf16_tile_rows() : attn_f32_tile_rows();
  const int Np = d->Tc * d->HW;
  a.tiles_per_chunk = (Np + QT - 1) / QT;
  a.tiles_last = (last_rows + QT - 1) / QT;
  a.tiles_per_head = (nch_launch - 1) * a.tiles_per_chunk + a.tiles_last;
  a.nblocks = d->B * d->H * a.tiles_per_head;
}

constexpr int kStateSegRows = 512;   // rows per segment for rehyat_state_update

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// streaming form (bf16): the window (tail + chunk) is gathered into K and V [nk_max][D]
// bf16 path: images of the linear-branch operands in the attention kernel's LDS layout,
// F*256 bytes per state (S^T) and per W (W^T).
size_t image_bytes(const rehyat_desc* d) { return (size_t)d->F * 256; }
size_t w_images_bytes(const rehyat_desc* d) {
  if (d->dtype != REHYAT_BF16 || phi_ahead(d)) return 0;
  return (size_t)(d->w_per_head ? d->H : 1) * image_bytes(d);
}

int64_t step_nk_max(const rehyat_desc* d) { return (int64_t)(d->Tc + d->To) * d->HW; }
size_t step_gather_bytes(const rehyat_desc* d) {
  if (d->dtype != REHYAT_BF16) return 0;
  return 2 * (size_t)d->B * d->H * (size_t)step_nk_max(d) * d->D * 2;
}

rehyat_status hybrid_fwd_impl(const rehyat_desc* d, const void* q, const void* k, const void* v,
                              const void* Wq, const void* Wk, void* y, float* lse, void* ws,
                              size_t ws_bytes, void* stream);

// Workspace of rehyat_hybrid_bwd, regions in this order (each rounded to 256 bytes).
struct BwdLayout {
  size_t part, states, gst, simg, gimg, wtq, wtk, dyb, gb, cvec, dvec, phiq, gq, gk, dws, dwz;
  size_t total;
};

BwdLayout bwd_layout(const rehyat_desc* d) {
  const size_t BH = (size_t)d->B * d->H, N = (size_t)d->T * d->HW, T = d->T;
  const size_t nch = n_chunks(d), E = state_elems(d), F = d->F, D = d->D;
  const size_t nW = d->w_per_head ? d->H : 1;
  const size_t sizes[16] = {BH * T * E * 4,   BH * nch * E * 4, BH * T * E * 4,  BH * nch * F * D * 2,
                            BH * T * F * D * 2, nW * F * D * 2,  nW * F * D * 2,  BH * N * D * 2,
                            BH * N * D * 2,   BH * N * 4,       BH * N * 4,      BH * N * F * 2,
                            BH * N * F * 2,   BH * N * F * 2,   BH * F * D * 4,  BH * F * 4};
  size_t off[16], o = 0;
  for (int i = 0; i < 16; ++i) {
    off[i] = o;
    o += (sizes[i] + 255) / 256 * 256;
  }
  BwdLayout L{off[0], off[1], off[2], off[3], off[4], off[5], off[6], off[7],
              off[8], off[9], off[10], off[11], off[12], off[13], off[14], off[15], o};
  return L;
}

}  // namespace

extern "C" {

const char* rehyat_status_str(rehyat_status s) {
  switch (s) {
    case REHYAT_OK: return "REHYAT_OK";
    case REHYAT_ERR_NULL: return "REHYAT_ERR_NULL";
    case REHYAT_ERR_SHAPE: return "REHYAT_ERR_SHAPE";
    case REHYAT_ERR_DTYPE: return "REHYAT_ERR_DTYPE";
    case REHYAT_ERR_ALIGN: return "REHYAT_ERR_ALIGN";
    case REHYAT_ERR_UNSUPPORTED: return "REHYAT_ERR_UNSUPPORTED";
    case REHYAT_ERR_WORKSPACE: return "REHYAT_ERR_WORKSPACE";
    case REHYAT_ERR_HIP: return "REHYAT_ERR_HIP";
    case REHYAT_ERR_ALIAS: return "REHYAT_ERR_ALIAS";
  }
  return "REHYAT_ERR_UNKNOWN";
}

const char* rehyat_last_error(void) { return g_err; }

rehyat_status rehyat_phi(const rehyat_desc* d, const void* x, int64_t n, const void* W, void* phi,
                         void* stream) {
  rehyat_status st = check_desc(d);
  if (st != REHYAT_OK) return st;
  if (n < 0) return fail(REHYAT_ERR_SHAPE, "n < 0");
  if (n == 0) return ok();
  if (!x || (needs_w(d) && !W) || !phi) return fail(REHYAT_ERR_NULL, "x, W and phi must be non-NULL");
  if (!aligned16(x) || !aligned16(W) || !aligned16(phi))
    return fail(REHYAT_ERR_ALIGN, "x, W, phi must be 16-byte aligned");
  const int64_t BH = (int64_t)d->B * d->H;
  if (BH * n * (d->D > d->F ? d->D : d->F) >= kMaxElems) return fail(REHYAT_ERR_SHAPE, "n too large");
  const size_t es = esize(d->dtype);
  if (overlaps(phi, BH * n * d->F * es, x, BH * n * d->D * es) ||
      overlaps(phi, BH * n * d->F * es, W, w_bytes(d)))
    return fail(REHYAT_ERR_ALIAS, "phi overlaps an input");
  hipStream_t s = (hipStream_t)stream;
  if (phi_ahead(d)) return hip_status(launch_phi_rows(d, x, n, W, phi, s), "rehyat_phi launch");
  const float us = 1.0f / std::sqrt((float)d->D);
  hipError_t e = (d->dtype == REHYAT_BF16)
                     ? launch_phi_bf16(x, n, W, d->w_per_head, d->H, (int)BH, d->F, phi, 0, us, s)
                     : launch_phi_f32(x, n, W, d->w_per_head, d->H, (int)BH, d->D, d->F, phi, us, s);
  return hip_status(e, "rehyat_phi launch");
}

size_t rehyat_state_update_workspace(const rehyat_desc* d, int64_t n) {
  if (check_desc(d) != REHYAT_OK || n <= 0) return 0;
  const int64_t nseg = (n + kStateSegRows - 1) / kStateSegRows;
  // per-segment partial states, then (maps evaluated ahead) the phi(k) rows
  return (size_t)d->B * d->H * nseg * state_elems(d) * sizeof(float) +
         (phi_ahead(d) ? phi_rows_bytes(d, n) : 0);
}

rehyat_status rehyat_state_update(const rehyat_desc* d, const void* k, const void* v, int64_t n,
                                  const void* Wk, float* S, float* z, void* ws, size_t ws_bytes,
                                  void* stream) {
  rehyat_status st = check_desc(d);
  if (st != REHYAT_OK) return st;
  if (n < 0) return fail(REHYAT_ERR_SHAPE, "n < 0");
  if (n == 0) return ok();
  if (!k || !v || (needs_w(d) && !Wk) || !S || !z)
    return fail(REHYAT_ERR_NULL, "k, v, Wk, S, z must be non-NULL");
  if (!aligned16(k) || !aligned16(v) || !aligned16(Wk) || !aligned16(S) || !aligned16(z))
    return fail(REHYAT_ERR_ALIGN, "pointers must be 16-byte aligned");
  const int64_t BH = (int64_t)d->B * d->H;
  if (BH * n * d->D >= kMaxElems) return fail(REHYAT_ERR_SHAPE, "n too large");
  const size_t need = rehyat_state_update_workspace(d, n);
  if (!ws || ws_bytes < need)
    return fail(REHYAT_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
  const size_t es = esize(d->dtype);
  const size_t nS = BH * d->F * d->D * sizeof(float), nz = BH * d->F * sizeof(float);
  const size_t nkv = BH * n * d->D * es;
  if (overlaps(S, nS, k, nkv) || overlaps(S, nS, v, nkv) || overlaps(z, nz, k, nkv) ||
      overlaps(z, nz, v, nkv) || overlaps(S, nS, z, nz) || overlaps(ws, need, S, nS) ||
      overlaps(ws, need, z, nz) || overlaps(ws, need, k, nkv) || overlaps(ws, need, v, nkv))
    return fail(REHYAT_ERR_ALIAS, "S, z, workspace and inputs must not overlap");
  StateArgs sa{};
  sa.ka = k; sa.va = v; sa.a_rows = n; sa.a_row0 = 0;
  sa.kb = k; sa.vb = v; sa.b_rows = n; sa.b_row0 = 0;
  sa.na = n; sa.n = n;
  sa.seg_len = kStateSegRows;
  sa.n_seg = (int)((n + kStateSegRows - 1) / kStateSegRows);
  sa.Wk = Wk; sa.w_per_head = d->w_per_head; sa.H = d->H;
  sa.part = reinterpret_cast<float*>(ws);
  sa.u_scale = 1.0f / std::sqrt((float)d->D);
  hipStream_t s = (hipStream_t)stream;
  if (phi_ahead(d)) {
    void* phik = reinterpret_cast<unsigned char*>(ws) + (size_t)BH * sa.n_seg * state_elems(d) * 4;
    hipError_t e = launch_phi_rows(d, k, n, Wk, phik, s);
    if (e != hipSuccess) return hip_status(e, "phi launch");
    sa.phik = phik; sa.phik_rows = n;
  }
  hipError_t e = launch_partial(d, sa, s);
  if (e != hipSuccess) return hip_status(e, "state partial launch");
  e = launch_fold_states(sa.part, sa.n_seg, S, z, d->F, d->D, 0, (int)BH, s);
  return hip_status(e, "state fold launch");
}

size_t rehyat_hybrid_fwd_workspace(const rehyat_desc* d) {
  if (check_desc(d) != REHYAT_OK) return 0;
  const size_t BH = (size_t)d->B * d->H;
  const size_t imgs = (d->dtype == REHYAT_BF16 && n_chunks(d) > 1)
                          ? BH * n_chunks(d) * image_bytes(d) + w_images_bytes(d) : 0;
  // maps evaluated ahead: phi(k) and phi(q) rows of the whole sequence
  const size_t phis = (phi_ahead(d) && n_chunks(d) > 1)
                          ? 2 * phi_rows_bytes(d, (int64_t)d->T * d->HW) : 0;
  // bf16: the persistent attention launch's work counters
  const size_t queue = d->dtype == REHYAT_BF16 ? kQueueBytes : 0;
  return BH * ((size_t)d->T + n_chunks(d)) * state_elems(d) * sizeof(float) + imgs + phis + queue;
}

rehyat_status rehyat_hybrid_fwd(const rehyat_desc* d, const void* q, const void* k, const void* v,
                                const void* Wq, const void* Wk, void* y, void* ws, size_t ws_bytes,
                                void* stream) {
  return hybrid_fwd_impl(d, q, k, v, Wq, Wk, y, nullptr, ws, ws_bytes, stream);
}

rehyat_status rehyat_hybrid_fwd_stats(const rehyat_desc* d, const void* q, const void* k,
                                      const void* v, const void* Wq, const void* Wk, void* y,
                                      float* lse, void* ws, size_t ws_bytes, void* stream) {
  if (!lse) return fail(REHYAT_ERR_NULL, "lse must be non-NULL");
  return hybrid_fwd_impl(d, q, k, v, Wq, Wk, y, lse, ws, ws_bytes, stream);
}

}  // extern "C"

namespace {

rehyat_status hybrid_fwd_impl(const rehyat_desc* d, const void* q, const void* k, const void* v,
                              const void* Wq, const void* Wk, void* y, float* lse, void* ws,
                              size_t ws_bytes, void* stream) {
  rehyat_status st = check_desc(d);
  if (st != REHYAT_OK) return st;
  if (!q || !k || !v || (needs_w(d) && (!Wq || !Wk)) || !y)
    return fail(REHYAT_ERR_NULL, "q, k, v, Wq, Wk, y must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(Wq) || !aligned16(Wk) ||
      !aligned16(y))
    return fail(REHYAT_ERR_ALIGN, "pointers must be 16-byte aligned");
  const size_t need = rehyat_hybrid_fwd_workspace(d);
  if (!ws || ws_bytes < need)
    return fail(REHYAT_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
  const int64_t N = (int64_t)d->T * d->HW;
  const int BH = d->B * d->H;
  const size_t es = esize(d->dtype);
  const size_t nin = (size_t)BH * N * d->D * es, ny = (size_t)BH * N * d->D * esize(d->y_dtype);
  const size_t nw = w_bytes(d);
  if (overlaps(y, ny, q, nin) || overlaps(y, ny, k, nin) || overlaps(y, ny, v, nin) ||
      overlaps(y, ny, Wq, nw) || overlaps(y, ny, Wk, nw) || overlaps(ws, need, y, ny) ||
      overlaps(ws, need, q, nin) || overlaps(ws, need, k, nin) || overlaps(ws, need, v, nin))
    return fail(REHYAT_ERR_ALIAS, "y, workspace and inputs must not overlap");
  if (lse) {
    const size_t nl = (size_t)BH * N * sizeof(float);
    if (!aligned16(lse)) return fail(REHYAT_ERR_ALIGN, "lse must be 16-byte aligned");
    if (overlaps(lse, nl, y, ny) || overlaps(lse, nl, q, nin) || overlaps(lse, nl, k, nin) ||
        overlaps(lse, nl, v, nin) || overlaps(lse, nl, ws, need))
      return fail(REHYAT_ERR_ALIAS, "lse must not overlap y, the inputs or the workspace");
  }

  hipStream_t s = (hipStream_t)stream;
  const int nch = n_chunks(d);
  const size_t E = state_elems(d);
  float* part = reinterpret_cast<float*>(ws);              // [BH][T][E]
  float* states = part + (size_t)BH * d->T * E;             // [BH][nch][E]
  unsigned char* simg = reinterpret_cast<unsigned char*>(states + (size_t)BH * nch * E);   // S^T images
  unsigned char* wimg = simg + (size_t)BH * nch * image_bytes(d);                 // W^T images
  unsigned char* phik = wimg + w_images_bytes(d);            // phi rows (maps evaluated ahead)
  unsigned char* phiq = phik + phi_rows_bytes(d, N);
  const float us = 1.0f / std::sqrt((float)d->D);
  const bool need_state = nch > 1;   // a single chunk has an empty linear set in both modes
  const bool bf16 = d->dtype == REHYAT_BF16;

  AttnArgs a{};
  a.q = q; a.q_rows = N; a.y = y;
  a.ka = k; a.va = v; a.a_rows = N;
  a.kb = k; a.vb = v; a.b_rows = N;
  a.Wq = Wq; a.w_per_head = d->w_per_head;
  a.S = states; a.z = states + (size_t)d->F * d->D;
  a.s_bh = (int64_t)nch * E; a.s_t = (int64_t)E; a.z_bh = a.s_bh; a.z_t = a.s_t;
  a.wt_img = wimg; a.wt_img_head = (int64_t)image_bytes(d);
  a.st_img = simg; a.st_img_bh = (int64_t)(nch * image_bytes(d)); a.st_img_t = (int64_t)image_bytes(d);
  a.phiq = (phi_ahead(d) && need_state) ? phiq : nullptr;
  a.lse = lse;
  a.H = d->H; a.HW = d->HW; a.Tc = d->Tc; a.To = d->To; a.T = d->T;
  a.n_chunks = nch; a.chunk0 = 0; a.step = 0;
  a.bidir = d->mode == REHYAT_BIDIR;
  a.y_f32 = d->y_dtype == REHYAT_F32;
  const int64_t Np = (int64_t)d->Tc * d->HW;
  fill_tiles(a, d, nch, (int)(N - (int64_t)(nch - 1) * Np));
  a.logit_scale = kLog2e / std::sqrt((float)d->D);
  a.u_scale = us;
  // the work counters of the persistent launch, the last kQueueBytes of the workspace: cleared
  // by the state scan's launch when there is one, else by a fill launch of their own
  if (bf16 && attn_bf16_persistent(a.nblocks))
    a.queue = reinterpret_cast<unsigned*>(reinterpret_cast<unsigned char*>(ws) + need - kQueueBytes);
  if (need_state) {
    StateArgs sa{};
    sa.ka = k; sa.va = v; sa.a_rows = N; sa.a_row0 = 0;
    sa.kb = k; sa.vb = v; sa.b_rows = N; sa.b_row0 = 0;
    sa.na = N; sa.n = N;
    sa.seg_len = d->HW;
    sa.n_seg = d->T;
    sa.Wk = Wk; sa.w_per_head = d->w_per_head; sa.H = d->H;
    sa.part = part;
    sa.u_scale = us;
    if (phi_ahead(d)) {
      hipError_t e = launch_phi_rows(d, k, N, Wk, phik, s);
      if (e == hipSuccess) e = launch_phi_rows(d, q, N, Wq, phiq, s);
      if (e != hipSuccess) return hip_status(e, "phi launch");
      sa.phik = phik; sa.phik_rows = N;
    }
    hipError_t e = launch_partial(d, sa, s);
    if (e != hipSuccess) return hip_status(e, "state partial launch");
    // the scan also writes the bf16 images of the linear branch and clears the counters
    e = launch_scan_states(part, states, d->F, d->D, d->T, d->Tc, d->To, nch,
                           d->mode == REHYAT_BIDIR, BH, bf16 ? simg : nullptr,
                           (int64_t)(nch * image_bytes(d)), (int64_t)image_bytes(d), Wq,
                           d->w_per_head ? d->H : 1, (bf16 && !phi_ahead(d)) ? wimg : nullptr,
                           a.queue, a.queue ? kAttnQueues : 0, s);
    if (e != hipSuccess) return hip_status(e, "state scan launch");
  }

  if (a.queue && !need_state) {
    hipError_t e = launch_zero_u32(a.queue, kAttnQueues, s);
    if (e != hipSuccess) return hip_status(e, "queue reset launch");
  }
  return hip_status(launch_attention(d, a, s), "attention launch");
}

// frames in chunk t
int step_frames(const rehyat_desc* d, int32_t t) {
  return (d->T - t * d->Tc) < d->Tc ? (d->T - t * d->Tc) : d->Tc;
}

// Argument checks of the recurrent step (both forms); need = the workspace size.
rehyat_status check_step(const rehyat_desc* d, int32_t t, const void* q_c, const void* k_c,
                         const void* v_c, const void* Wq, const void* Wk, const float* S,
                         const float* z, const void* k_tail, const void* v_tail, const void* y_c,
                         const void* ws, size_t ws_bytes, size_t need,
                         bool static_ws = false) {
  if (d->To > d->Tc) return fail(REHYAT_ERR_UNSUPPORTED, "recurrent step needs To <= Tc");
  const int nch = n_chunks(d);
  if (t < 0 || t >= nch) return fail(REHYAT_ERR_SHAPE, "chunk_index %d outside [0, %d)", t, nch);
  const int cf = step_frames(d, t);
  if (cf < d->To) return fail(REHYAT_ERR_UNSUPPORTED, "final chunk of %d frames is shorter than To = %d", cf, d->To);
  if (!q_c || !k_c || !v_c || (needs_w(d) && (!Wq || !Wk)) || !S || !z || !y_c)
    return fail(REHYAT_ERR_NULL, "q_c, k_c, v_c, Wq, Wk, S, z, y_c must be non-NULL");
  if (d->To > 0 && (!k_tail || !v_tail)) return fail(REHYAT_ERR_NULL, "k_tail, v_tail needed when To > 0");
  if (!aligned16(q_c) || !aligned16(k_c) || !aligned16(v_c) || !aligned16(Wq) || !aligned16(Wk) ||
      !aligned16(S) || !aligned16(z) || !aligned16(y_c) ||
      (d->To > 0 && (!aligned16(k_tail) || !aligned16(v_tail))))
    return fail(REHYAT_ERR_ALIGN, "pointers must be 16-byte aligned");
  if (!static_ws) {   // (the static scratch array is an allocation of its own)
    if (!ws || ws_bytes < need)
      return fail(REHYAT_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
    if (!aligned16(ws)) return fail(REHYAT_ERR_ALIGN, "workspace must be 16-byte aligned");
  }
  const int BH = d->B * d->H;
  const int64_t crow = (int64_t)cf * d->HW;          // rows in this chunk
  const int64_t trow = (int64_t)d->To * d->HW;       // rows in the tail
  const size_t es = esize(d->dtype);
  const size_t nc = (size_t)BH * crow * d->D * es, nt = (size_t)BH * trow * d->D * es;
  const size_t ny = (size_t)BH * crow * d->D * esize(d->y_dtype);
  const size_t nS = (size_t)BH * d->F * d->D * 4, nz = (size_t)BH * d->F * 4;
  const void* ins[3] = {q_c, k_c, v_c};
  for (const void* p : ins) {
    if (overlaps(y_c, ny, p, nc) || overlaps(S, nS, p, nc) || overlaps(z, nz, p, nc) ||
        overlaps(k_tail, nt, p, nc) || overlaps(v_tail, nt, p, nc) || overlaps(ws, need, p, nc))
      return fail(REHYAT_ERR_ALIAS, "outputs must not overlap the chunk inputs");
  }
  if (overlaps(S, nS, z, nz) || overlaps(y_c, ny, S, nS) || overlaps(y_c, ny, z, nz) ||
      overlaps(k_tail, nt, v_tail, nt) || overlaps(y_c, ny, k_tail, nt) ||
      overlaps(y_c, ny, v_tail, nt) || overlaps(ws, need, S, nS) || overlaps(ws, need, z, nz) ||
      overlaps(ws, need, y_c, ny) || overlaps(ws, need, k_tail, nt) || overlaps(ws, need, v_tail, nt))
    return fail(REHYAT_ERR_ALIAS, "outputs and workspace must not overlap");
  return ok();
}

}  // namespace


extern "C" {

size_t rehyat_recurrent_step_workspace(const rehyat_desc* d) {
  if (check_desc(d) != REHYAT_OK) return 0;
  const size_t imgs = (d->dtype == REHYAT_BF16)
                          ? (size_t)d->B * d->H * image_bytes(d) + w_images_bytes(d) : 0;
  // maps evaluated ahead: phi(q) of the chunk and phi(k) of the gathered window
  const size_t phis = phi_ahead(d) ? phi_rows_bytes(d, (int64_t)d->Tc * d->HW) +
                                         phi_rows_bytes(d, step_nk_max(d))
                                   : 0;
  return (size_t)d->B * d->H * d->Tc * state_elems(d) * sizeof(float) + step_gather_bytes(d) +
         imgs + phis;
}

rehyat_status rehyat_recurrent_step(const rehyat_desc* d, int32_t t, const void* q_c,
                                    const void* k_c, const void* v_c, const void* Wq,
                                    const void* Wk, float* S, float* z, void* k_tail, void* v_tail,
                                    void* y_c, void* ws, size_t ws_bytes, void* stream) {
  rehyat_status st = check_desc(d);
  if (st != REHYAT_OK) return st;
  const size_t need = rehyat_recurrent_step_workspace(d);
  st = check_step(d, t, q_c, k_c, v_c, Wq, Wk, S, z, k_tail, v_tail, y_c, ws, ws_bytes, need);
  if (st != REHYAT_OK) return st;
  const int BH = d->B * d->H;
  const int cf = step_frames(d, t);
  const int64_t crow = (int64_t)cf * d->HW;          // rows in this chunk
  const int64_t trow = (int64_t)d->To * d->HW;       // rows in the tail
  const size_t es = esize(d->dtype);

  hipStream_t s = (hipStream_t)stream;
  const float us = 1.0f / std::sqrt((float)d->D);
  const int64_t tail_in = (t > 0) ? trow : 0;        // tail rows in the window

  // 1. attention over window = tail + chunk, linear branch from the carried state
  AttnArgs a{};
  a.q = q_c; a.q_rows = crow; a.y = y_c;
  a.ka = k_tail ? k_tail : k_c; a.va = v_tail ? v_tail : v_c; a.a_rows = k_tail ? trow : crow;
  a.kb = k_c; a.vb = v_c; a.b_rows = crow;
  float* part = reinterpret_cast<float*>(ws);
  void* phiq_step = nullptr;   // phi(q_c) rows (maps evaluated ahead)
  void* phik_step = nullptr;   // phi rows of the gathered window keys
  void* kwin_step = nullptr;
  if (d->dtype == REHYAT_BF16) {
    // gather the window contiguously: K and V [nk_max][D] per head
    uint16_t* kwin = reinterpret_cast<uint16_t*>(part + (size_t)BH * d->Tc * state_elems(d));
    uint16_t* vwin = kwin + (size_t)BH * step_nk_max(d) * d->D;
    // images of the carried state S^T and of W^T for the linear branch
    unsigned char* simg = reinterpret_cast<unsigned char*>(part + (size_t)BH * d->Tc * state_elems(d)) +
                          step_gather_bytes(d);
    unsigned char* wimg = simg + (size_t)BH * image_bytes(d);
    phiq_step = wimg + w_images_bytes(d);
    phik_step = reinterpret_cast<unsigned char*>(phiq_step) + phi_rows_bytes(d, (int64_t)d->Tc * d->HW);
    if (t > 0) {
      hipError_t ei = launch_linear_images_bf16(S, (int64_t)d->F * d->D, 0, 1, BH, d->F, simg,
                                                (int64_t)image_bytes(d), 0, Wq,
                                                d->w_per_head ? d->H : 1,
                                                phi_ahead(d) ? nullptr : wimg, nullptr, 0, s);
      if (ei != hipSuccess) return hip_status(ei, "linear image launch");
      if (phi_ahead(d)) {
        ei = launch_phi_rows(d, q_c, crow, Wq, phiq_step, s);
        if (ei != hipSuccess) return hip_status(ei, "phi launch");
        a.phiq = phiq_step;
      }
    }
    a.wt_img = wimg; a.wt_img_head = (int64_t)image_bytes(d);
    a.st_img = simg; a.st_img_bh = (int64_t)image_bytes(d); a.st_img_t = 0;
    hipError_t e = launch_gather_window_bf16(a.ka, a.va, a.a_rows, a.a_rows - tail_in, k_c, v_c,
                                             crow, tail_in, tail_in + crow, kwin, vwin,
                                             step_nk_max(d), BH, s);
    if (e != hipSuccess) return hip_status(e, "window gather launch");
    a.ka = kwin; a.va = vwin; a.a_rows = step_nk_max(d);
    kwin_step = kwin;
  }
  a.Wq = Wq; a.w_per_head = d->w_per_head;
  a.S = S; a.z = z;
  a.s_bh = (int64_t)d->F * d->D; a.s_t = 0; a.z_bh = d->F; a.z_t = 0;
  a.H = d->H; a.HW = d->HW; a.Tc = d->Tc; a.To = d->To; a.T = d->T;
  a.n_chunks = 1; a.chunk0 = t; a.step = 1; a.bidir = 0;
  a.y_f32 = d->y_dtype == REHYAT_F32;
  fill_tiles(a, d, 1, (int)crow);
  a.logit_scale = kLog2e / std::sqrt((float)d->D);
  a.u_scale = us;
  hipError_t e = launch_attention(d, a, s);
  if (e != hipSuccess) return hip_status(e, "attention launch");

  // 2. fold the window rows that no later window reaches (all but the last To frames)
  const int64_t nfold = tail_in + crow - trow;
  if (nfold > 0) {
    StateArgs sa{};
    sa.ka = k_tail ? k_tail : k_c; sa.va = v_tail ? v_tail : v_c;
    sa.a_rows = k_tail ? trow : crow; sa.a_row0 = 0;
    sa.kb = k_c; sa.vb = v_c; sa.b_rows = crow; sa.b_row0 = 0;
    sa.na = tail_in; sa.n = nfold;
    sa.seg_len = d->HW;
    sa.n_seg = (int)((nfold + d->HW - 1) / d->HW);
    sa.Wk = Wk; sa.w_per_head = d->w_per_head; sa.H = d->H;
    sa.part = part;
    sa.u_scale = us;
    if (phi_ahead(d)) {
      // phi of the gathered window keys (tail rows, then chunk rows: the fold's row order;
      // all nk_max rows of each head's window buffer, of which the first nfold are used)
      e = launch_phi_rows(d, kwin_step, step_nk_max(d), Wk, phik_step, s);
      if (e != hipSuccess) return hip_status(e, "phi launch");
      sa.phik = phik_step; sa.phik_rows = step_nk_max(d);
    }
    e = launch_partial(d, sa, s);
    if (e != hipSuccess) return hip_status(e, "state partial launch");
    e = launch_fold_states(part, sa.n_seg, S, z, d->F, d->D, t == 0, BH, s);
    if (e != hipSuccess) return hip_status(e, "state fold launch");
  } else if (t == 0) {
    e = launch_fold_states(part, 0, S, z, d->F, d->D, 1, BH, s);   // empty state
    if (e != hipSuccess) return hip_status(e, "state init launch");
  }

  // 3. the chunk's last To frames become the tail
  if (trow > 0) {
    e = launch_copy_rows(k_c, v_c, k_tail, v_tail, crow, crow - trow, trow, (int)(d->D * es), BH, s);
    if (e != hipSuccess) return hip_status(e, "tail copy launch");
  }
  return ok();
}

size_t rehyat_recurrent_step_fused_workspace(const rehyat_desc* d) {
  if (check_desc(d) != REHYAT_OK) return 0;
  const size_t BH = (size_t)d->B * d->H;
  // completion counters, then the new state and two frames' partials per head
  return round_up((int64_t)(BH * sizeof(unsigned)), 256) + 3 * BH * state_elems(d) * sizeof(float);
}

}  // extern "C"

namespace {

// The single-launch step on the scratch buffer ws (its counters zero on entry, left zero).
rehyat_status device_scratch(hipStream_t s, void** out);

// static_ws: every argument is checked first, then ws is the current device's static array.
rehyat_status step_fused_impl(const rehyat_desc* d, int32_t t, const void* q_c, const void* k_c,
                              const void* v_c, const void* Wq, const void* Wk, float* S, float* z,
                              const void* k_tail, const void* v_tail, void* k_tail_out,
                              void* v_tail_out, void* y_c, void* ws, size_t ws_bytes,
                              void* stream, bool static_ws = false) {
  rehyat_status st = check_desc(d);
  if (st != REHYAT_OK) return st;
  if (d->dtype != REHYAT_BF16 || d->phi_kind != REHYAT_PHI_POLY2)
    return fail(REHYAT_ERR_UNSUPPORTED,
                "the single-launch step supports bf16 inputs with the fixed feature map");
  const size_t need = rehyat_recurrent_step_fused_workspace(d);
  if (static_ws && need > (size_t)REHYAT_STATIC_SCRATCH_BYTES)
    return fail(REHYAT_ERR_WORKSPACE,
                "the step needs %zu bytes of scratch, beyond the static %d bytes "
                "(use rehyat_recurrent_step_fused with a workspace)",
                need, REHYAT_STATIC_SCRATCH_BYTES);
  st = check_step(d, t, q_c, k_c, v_c, Wq, Wk, S, z, k_tail, v_tail, y_c, ws, ws_bytes, need,
                  static_ws);
  if (st != REHYAT_OK) return st;
  const int BH = d->B * d->H;
  const int64_t crow = (int64_t)step_frames(d, t) * d->HW;   // rows in this chunk
  const int64_t trow = (int64_t)d->To * d->HW;               // rows in the tail
  const int64_t tail_in = (t > 0) ? trow : 0;                // tail rows in the window
  if (d->To > 0) {
    // the new tail: its own buffers, apart from everything else the call touches
    if (!k_tail_out || !v_tail_out)
      return fail(REHYAT_ERR_NULL, "k_tail_out, v_tail_out needed when To > 0");
    if (!aligned16(k_tail_out) || !aligned16(v_tail_out))
      return fail(REHYAT_ERR_ALIGN, "pointers must be 16-byte aligned");
    const size_t es = esize(d->dtype);
    const size_t nt = (size_t)BH * trow * d->D * es, nc = (size_t)BH * crow * d->D * es;
    const size_t ny = (size_t)BH * crow * d->D * esize(d->y_dtype);
    const size_t nS = (size_t)BH * d->F * d->D * 4, nz = (size_t)BH * d->F * 4;
    const void* other[9] = {q_c, k_c, v_c, k_tail, v_tail, y_c, S, z, ws};
    const size_t other_n[9] = {nc, nc, nc, nt, nt, ny, nS, nz, need};
    for (void* o : {k_tail_out, v_tail_out})
      for (int i = 0; i < 9; ++i)
        if (overlaps(o, nt, other[i], other_n[i]))
          return fail(REHYAT_ERR_ALIAS, "k_tail_out, v_tail_out must not overlap the other buffers");
    if (overlaps(k_tail_out, nt, v_tail_out, nt))
      return fail(REHYAT_ERR_ALIAS, "k_tail_out and v_tail_out must not overlap");
  }
  if (static_ws) {
    st = device_scratch((hipStream_t)stream, &ws);
    if (st != REHYAT_OK) return st;
  }
  const size_t E = state_elems(d);
  unsigned* counter = reinterpret_cast<unsigned*>(ws);
  float* xs = reinterpret_cast<float*>(reinterpret_cast<unsigned char*>(ws) +
                                       round_up((int64_t)(BH * sizeof(unsigned)), 256));
  const float us = 1.0f / std::sqrt((float)d->D);

  AttnArgs a{};
  a.q = q_c; a.q_rows = crow; a.y = y_c;
  a.ka = k_tail ? k_tail : k_c; a.va = v_tail ? v_tail : v_c; a.a_rows = k_tail ? trow : crow;
  a.kb = k_c; a.vb = v_c; a.b_rows = crow;
  a.Wq = Wq; a.w_per_head = d->w_per_head;
  a.S = S; a.z = z;
  a.s_bh = (int64_t)d->F * d->D; a.s_t = 0; a.z_bh = d->F; a.z_t = 0;
  a.H = d->H; a.HW = d->HW; a.Tc = d->Tc; a.To = d->To; a.T = d->T;
  a.n_chunks = 1; a.chunk0 = t; a.step = 1; a.bidir = 0;
  a.y_f32 = d->y_dtype == REHYAT_F32;
  fill_tiles(a, d, 1, (int)crow);
  a.logit_scale = kLog2e / std::sqrt((float)d->D);
  a.u_scale = us;

  StepArgs sp{};
  // the window rows that no later window reaches (all but the last To frames), per frame
  const int64_t nfold = tail_in + crow - trow;
  StateArgs& sa = sp.fold;
  sa.ka = a.ka; sa.va = a.va; sa.a_rows = a.a_rows; sa.a_row0 = 0;
  sa.kb = k_c; sa.vb = v_c; sa.b_rows = crow; sa.b_row0 = 0;
  sa.na = tail_in; sa.n = nfold;
  sa.seg_len = d->HW;
  sa.n_seg = (int)((nfold + d->HW - 1) / d->HW);
  sa.Wk = Wk; sa.w_per_head = d->w_per_head; sa.H = d->H;
  sa.u_scale = us;
  sp.fold_blocks = (int)round_up(BH, 8);
  sp.per_head = a.tiles_per_head + 1;
  sp.counter = counter;
  sp.xs = xs;
  sp.pp = xs + (size_t)BH * E;
  sp.S = S; sp.z = z;
  sp.init = t == 0;
  sp.kc = k_c; sp.vc = v_c; sp.crow = crow;
  sp.ktail = k_tail_out; sp.vtail = v_tail_out; sp.trow = d->To > 0 ? trow : 0;
  hipStream_t s = (hipStream_t)stream;
  timed_begin(s, 4);
  const hipError_t e = launch_step_bf16(a, sp, d->F, s);
  timed_end(s, 4);
  return hip_status(e, "step launch");
}

// ---- scratch without an allocation ------------------------------------------------------
// The step's scratch (completion counters, the new state, the fold's partials) for
// rehyat_recurrent_step_fused_noalloc lives in this array: one copy on every device the
// library runs on, resident until the process ends. Host code never uses the array's name
// as an address: the device address of each device's copy comes from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[REHYAT_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

__global__ void zero_scratch_kernel(u32x4* p, int64_t n16) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = u32x4{0u, 0u, 0u, 0u};
}

// Device address of the current device's scratch array. The first call on a device looks
// it up (with that device current) and enqueues a fill kernel on `s` that zeroes the whole
// array, so that the completion counters start at zero; later calls leave them zero.
rehyat_status device_scratch(hipStream_t s, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(REHYAT_ERR_UNSUPPORTED, "device %d beyond the %d devices supported", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(REHYAT_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    const int64_t n16 = REHYAT_STATIC_SCRATCH_BYTES / 16;
    hipLaunchKernelGGL(zero_scratch_kernel, dim3(256), dim3(256), 0, s,
                       reinterpret_cast<u32x4*>(p), n16);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_status(e, "scratch fill launch");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ok();
}

}  // namespace

extern "C" {

rehyat_status rehyat_recurrent_step_fused(const rehyat_desc* d, int32_t t, const void* q_c,
                                          const void* k_c, const void* v_c, const void* Wq,
                                          const void* Wk, float* S, float* z, const void* k_tail,
                                          const void* v_tail, void* k_tail_out, void* v_tail_out,
                                          void* y_c, void* ws, size_t ws_bytes, void* stream) {
  return step_fused_impl(d, t, q_c, k_c, v_c, Wq, Wk, S, z, k_tail, v_tail, k_tail_out,
                         v_tail_out, y_c, ws, ws_bytes, stream);
}

rehyat_status rehyat_recurrent_step_fused_noalloc(const rehyat_desc* d, int32_t t,
                                                  const void* q_c, const void* k_c,
                                                  const void* v_c, const void* Wq, const void* Wk,
                                                  float* S, float* z, const void* k_tail,
                                                  const void* v_tail, void* k_tail_out,
                                                  void* v_tail_out, void* y_c, void* stream) {
  return step_fused_impl(d, t, q_c, k_c, v_c, Wq, Wk, S, z, k_tail, v_tail, k_tail_out,
                         v_tail_out, y_c, nullptr, REHYAT_STATIC_SCRATCH_BYTES, stream, true);
}

size_t rehyat_hybrid_bwd_workspace(const rehyat_desc* d) {
  if (check_desc(d) != REHYAT_OK) return 0;
  return bwd_layout(d).total;
}

rehyat_status rehyat_hybrid_bwd(const rehyat_desc* d, const void* q, const void* k, const void* v,
                                const void* Wq, const void* Wk, const void* y, const float* lse,
                                const void* dy, float* dq, float* dk, float* dv, float* dWq,
                                float* dWk, void* ws, size_t ws_bytes, void* stream) {
  rehyat_status st = check_desc(d);
  if (st != REHYAT_OK) return st;
  if (d->dtype != REHYAT_BF16 || d->phi_kind != REHYAT_PHI_POLY2)
    return fail(REHYAT_ERR_UNSUPPORTED, "the backward supports bf16 inputs with the fixed feature map");
  if (d->mode != REHYAT_CAUSAL)
    return fail(REHYAT_ERR_UNSUPPORTED, "the backward supports the causal form");
  const void* ins[8] = {q, k, v, Wq, Wk, y, lse, dy};
  const void* outs[5] = {dq, dk, dv, dWq, dWk};
  for (const void* p : ins)
    if (!p) return fail(REHYAT_ERR_NULL, "q, k, v, Wq, Wk, y, lse, dy must be non-NULL");
  for (const void* p : outs)
    if (!p) return fail(REHYAT_ERR_NULL, "dq, dk, dv, dWq, dWk must be non-NULL");
  for (const void* p : ins)
    if (!aligned16(p)) return fail(REHYAT_ERR_ALIGN, "pointers must be 16-byte aligned");
  for (const void* p : outs)
    if (!aligned16(p)) return fail(REHYAT_ERR_ALIGN, "pointers must be 16-byte aligned");
  const BwdLayout L = bwd_layout(d);
  if (!ws || ws_bytes < L.total)
    return fail(REHYAT_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", L.total, ws_bytes);
  const int BH = d->B * d->H;
  const int64_t N = (int64_t)d->T * d->HW;
  const int F = d->F, D = d->D, T = d->T, nch = n_chunks(d);
  const size_t nin = (size_t)BH * N * D * 2, nyb = (size_t)BH * N * D * esize(d->y_dtype);
  const size_t nd = (size_t)BH * N * D * 4, nl = (size_t)BH * N * 4;
  const size_t nwb = w_bytes(d), nwo = (size_t)(d->w_per_head ? d->H : 1) * D * F * 4;
  const void* in_p[8] = {q, k, v, Wq, Wk, y, lse, dy};
  const size_t in_n[8] = {nin, nin, nin, nwb, nwb, nyb, nl, nyb};
  void* out_p[6] = {dq, dk, dv, dWq, dWk, ws};
  const size_t out_n[6] = {nd, nd, nd, nwo, nwo, L.total};
  for (int i = 0; i < 6; ++i) {
    for (int j = 0; j < 8; ++j)
      if (overlaps(out_p[i], out_n[i], in_p[j], in_n[j]))
        return fail(REHYAT_ERR_ALIAS, "outputs and workspace must not overlap the inputs");
    for (int j = i + 1; j < 6; ++j)
      if (overlaps(out_p[i], out_n[i], out_p[j], out_n[j]))
        return fail(REHYAT_ERR_ALIAS, "outputs and workspace must not overlap each other");
  }

  hipStream_t s = (hipStream_t)stream;
  unsigned char* w8 = reinterpret_cast<unsigned char*>(ws);
  float* part = reinterpret_cast<float*>(w8 + L.part);
  float* states = reinterpret_cast<float*>(w8 + L.states);
  float* gst = reinterpret_cast<float*>(w8 + L.gst);
  uint16_t* simg = reinterpret_cast<uint16_t*>(w8 + L.simg);
  uint16_t* gimg = reinterpret_cast<uint16_t*>(w8 + L.gimg);
  uint16_t* wtq = reinterpret_cast<uint16_t*>(w8 + L.wtq);
  uint16_t* wtk = reinterpret_cast<uint16_t*>(w8 + L.wtk);
  uint16_t* dyb = reinterpret_cast<uint16_t*>(w8 + L.dyb);
  uint16_t* gb = reinterpret_cast<uint16_t*>(w8 + L.gb);
  float* cvec = reinterpret_cast<float*>(w8 + L.cvec);
  float* dvec = reinterpret_cast<float*>(w8 + L.dvec);
  uint16_t* phiq = reinterpret_cast<uint16_t*>(w8 + L.phiq);
  uint16_t* gq = reinterpret_cast<uint16_t*>(w8 + L.gq);
  uint16_t* gk = reinterpret_cast<uint16_t*>(w8 + L.gk);
  float* dws = reinterpret_cast<float*>(w8 + L.dws);
  float* dwz = reinterpret_cast<float*>(w8 + L.dwz);
  const int64_t E = (int64_t)state_elems(d);
  const float us = 1.0f / std::sqrt((float)D);
  const int nW = d->w_per_head ? d->H : 1;
  hipError_t e;
#define REHYAT_TRY(call, what) \
  do {                         \
    e = (call);                \
    if (e != hipSuccess) return hip_status(e, what); \
  } while (0)

  // 1. forward states S_t, z_t of every chunk (as in the forward)
  {
    StateArgs sa{};
    sa.ka = k; sa.va = v; sa.a_rows = N; sa.a_row0 = 0;
    sa.kb = k; sa.vb = v; sa.b_rows = N; sa.b_row0 = 0;
    sa.na = N; sa.n = N; sa.seg_len = d->HW; sa.n_seg = T;
    sa.Wk = Wk; sa.w_per_head = d->w_per_head; sa.H = d->H;
    sa.part = part; sa.u_scale = us;
    REHYAT_TRY(launch_partial(d, sa, s), "state partial launch");
    REHYAT_TRY(launch_scan_states(part, states, F, D, T, d->Tc, d->To, nch, 0, BH, nullptr, 0, 0,
                                  nullptr, 0, nullptr, nullptr, 0, s),
               "state scan launch");
    REHYAT_TRY(launch_state_rows_bf16(states, nch * E, E, nch, BH, F, simg, s), "state image launch");
  }
  REHYAT_TRY(launch_transpose_w(Wq, F, nW, wtq, s), "transpose launch");
  REHYAT_TRY(launch_transpose_w(Wk, F, nW, wtk, s), "transpose launch");
  // 2. per-row dy.y, dy / den
  REHYAT_TRY(launch_bwd_prep(y, dy, d->y_dtype == REHYAT_F32, lse, (int64_t)BH * N, us, dyb, gb, cvec, dvec, s),
             "prep launch");
  // 3. dq (window and linear read-out), phi(q) and gq rows
  BwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.dyb = dyb; a.gb = gb; a.lse = lse; a.cvec = cvec; a.dvec = dvec;
  a.w_per_head = d->w_per_head;
  a.H = d->H; a.HW = d->HW; a.Tc = d->Tc; a.To = d->To; a.T = T; a.N = (int)N; a.n_chunks = nch;
  a.logit_scale = kLog2e * us; a.u_scale = us;
  const int64_t Np = (int64_t)d->Tc * d->HW;
  const int last_rows = (int)(N - (int64_t)(nch - 1) * Np);
  {
    BwdArgs b = a;
    b.w = reinterpret_cast<const uint16_t*>(Wq); b.wt = wtq;
    b.st_img = simg; b.st = states; b.nslot = nch;
    b.dx = dq; b.phi_out = phiq; b.g_out = gq;
    b.tiles_per_chunk = (int)((Np + 255) / 256);
    b.tiles_last = (last_rows + 255) / 256;
    b.tiles_per_head = (nch - 1) * b.tiles_per_chunk + b.tiles_last;
    timed_begin(s, 3);
    e = launch_bwd_dq(b, F, BH * b.tiles_per_head, s);
    timed_end(s, 3);
    if (e != hipSuccess) return hip_status(e, "dq launch");
  }
  // 4. reverse states: per query frame sums phi(q) g^T and phi(q) c, suffix over chunks
  {
    StateArgs sa{};
    sa.ka = gb; sa.va = gb; sa.a_rows = N; sa.a_row0 = 0;
    sa.kb = gb; sa.vb = gb; sa.b_rows = N; sa.b_row0 = 0;
    sa.na = N; sa.n = N; sa.seg_len = d->HW; sa.n_seg = T;
    sa.part = part; sa.phik = phiq; sa.phik_rows = N; sa.zw = cvec;
    REHYAT_TRY(launch_state_partial_phi_bf16(sa, F, BH, s), "reverse state launch");
    REHYAT_TRY(launch_suffix_states(part, gst, F, D, T, d->Tc, d->To, BH, s), "suffix launch");
    REHYAT_TRY(launch_state_rows_bf16(gst, T * E, E, T, BH, F, gimg, s), "state image launch");
  }
  // 5. dk, dv (window and linear parts), gk rows
  {
    BwdArgs b = a;
    b.w = reinterpret_cast<const uint16_t*>(Wk); b.wt = wtk;
    b.st_img = gimg; b.st = gst; b.nslot = T;
    b.dx = dk; b.dv = dv; b.g_out = gk;
    b.tiles_per_chunk = (int)((Np + 127) / 128);
    b.tiles_last = (last_rows + 127) / 128;
    b.tiles_per_head = (nch - 1) * b.tiles_per_chunk + b.tiles_last;
    timed_begin(s, 2);
    e = launch_bwd_dkdv(b, F, BH * b.tiles_per_head, s);
    timed_end(s, 2);
    if (e != hipSuccess) return hip_status(e, "dk/dv launch");
  }
  // 6. dW = sum over rows of x gx^T (per frame, folded per head, summed over heads / batch)
  for (int side = 0; side < 2; ++side) {
    StateArgs sa{};
    const void* x = side ? k : q;
    sa.ka = x; sa.va = x; sa.a_rows = N; sa.a_row0 = 0;
    sa.kb = x; sa.vb = x; sa.b_rows = N; sa.b_row0 = 0;
    sa.na = N; sa.n = N; sa.seg_len = d->HW; sa.n_seg = T;
    sa.part = part; sa.phik = side ? gk : gq; sa.phik_rows = N;
    REHYAT_TRY(launch_state_partial_phi_bf16(sa, F, BH, s), "dW partial launch");
    REHYAT_TRY(launch_fold_states(part, T, dws, dwz, F, D, 1, BH, s), "dW fold launch");
    REHYAT_TRY(launch_dw_finalize(dws, (int64_t)F * D, BH, d->H, d->w_per_head, F, side ? dWk : dWq, s),
               "dW finalize launch");
  }
#undef REHYAT_TRY
  return ok();
}

rehyat_status rehyat_timing_enable(int32_t enable) {
  if (enable && !g_timing.created) {
    for (int i = 0; i < 2 * kMaxTimed; ++i) {
      hipError_t e = hipEventCreate(&g_timing.ev[i]);
      if (e != hipSuccess) return hip_status(e, "hipEventCreate");
    }
    g_timing.created = true;
  }
  if (enable < 0 || enable > 4) return fail(REHYAT_ERR_SHAPE, "timing selector %d unknown", enable);
  g_timing.enabled = enable != 0;
  g_timing.which = enable;
  g_timing.count = 0;
  return ok();
}

rehyat_status rehyat_timing_read(double* total_ms, int64_t* launches) {
  if (!total_ms || !launches) return fail(REHYAT_ERR_NULL, "outputs must be non-NULL");
  *total_ms = 0.0;
  *launches = g_timing.count;
  if (g_timing.count > 0) {
    hipError_t e = hipEventSynchronize(g_timing.ev[2 * g_timing.count - 1]);
    if (e != hipSuccess) return hip_status(e, "hipEventSynchronize");
    for (int i = 0; i < g_timing.count; ++i) {
      float ms = 0.0f;
      e = hipEventElapsedTime(&ms, g_timing.ev[2 * i], g_timing.ev[2 * i + 1]);
      if (e != hipSuccess) return hip_status(e, "hipEventElapsedTime");
      *total_ms += ms;
    }
  }
  g_timing.count = 0;
  return ok();
}

}  // extern "C"
