// C ABI of the PISA forward pass: argument validation, workspace layout and
// launch order. Every check runs before anything is enqueued.
#include <math.h>
#include <string.h>

#include <mutex>

#include "../../include/pisa.h"
#include "pisa_internal.h"

#define PISA_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_last_hip_error[256] = "";

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Rows longer than kRouteMaxBlocks blocks go through a score buffer in the
// workspace. One pass of pisa_select holds the scores of this many heads:
// enough for about 2048 workgroups of the score kernel (128 x 128 score
// tiles), at most all of them. The buffer is sized for one such chunk, about
// 2048 x 128² fp64 values (256 MiB) whatever the head count (one head's n²
// scores when that alone is more).
long route_chunk(long bh, long n) {
  const long t = n >= 512 ? (n + 127) / 128 : (n + 63) / 64;
  const long c = (2048 + t * t - 1) / (t * t);
  return c < 1 ? 1 : (c > bh ? bh : c);
}

// Validates the shape; fills the workspace layout. Returns PISA_OK or the error.
pisa_status_t check_shape(const pisa_shape_t* s, pisa::WsLayout* w) {
  if (s == nullptr) return PISA_EINVAL;
  if (s->B < 1 || s->H < 1 || s->L < 1 || s->D < 1 || s->block < 1) return PISA_EINVAL;
  if (s->dtype != PISA_F32 && s->dtype != PISA_BF16) return PISA_EINVAL;
  if (s->layout != PISA_LAYOUT_BHLD && s->layout != PISA_LAYOUT_BLHD) return PISA_EINVAL;
  if (s->D != 64 && s->D != 128) return PISA_ENOTSUP;
  if (s->block != 64 && s->block != 128) return PISA_ENOTSUP;
  const long bh = (long)s->B * s->H;
  const long n = ((long)s->L + s->block - 1) / s->block;
  if (n > pisa::kMaxBlocks) return PISA_ENOTSUP;
  if (bh > (1L << 24)) return PISA_ENOTSUP;  // grid sizes stay far inside 2^31
  if (bh * n * (s->block / 64) > (1L << 30)) return PISA_ENOTSUP;
  if (w == nullptr) return PISA_OK;
  const int esz = s->dtype == PISA_BF16 ? 2 : 4;
  w->bh = bh;
  w->n = (int)n;
  w->spb = s->block / 64;
  w->nct = (int)((n + 63) / 64);
  // Statistics run over runs of cb consecutive blocks, one workgroup each: up
  // to 1024 tokens, fewer when that would leave fewer than ~512 workgroups to
  // spread over the chip (short sequences).
  const long cb_max = 1024 / s->block, by_size = bh * n / 512;
  w->cb = (int)(by_size < 1 ? 1 : (by_size > cb_max ? cb_max : by_size));
  w->nch = (int)((n + w->cb - 1) / w->cb);
  w->esz = esz;
  const size_t sub = (size_t)64 * s->D * esz;
  size_t off = 0;
  w->kp = off;
  off = align256(off + (size_t)bh * n * w->spb * sub);
  w->vp = off;
  off = align256(off + (size_t)bh * n * w->spb * sub);
  w->kmax2 = off;
  off = align256(off + (size_t)bh * w->nch * sizeof(float));
  w->redo = off;
  off = align256(off + ((size_t)bh * n * w->spb + 1) * sizeof(int32_t));
  w->sync = off;
  off = align256(off + pisa::kSyncCounters * sizeof(int32_t));
  w->dense_total = off;
  w->kbp = off;
  off = align256(off + (size_t)bh * w->nct * sub);
  w->vbp = off;
  off = align256(off + (size_t)bh * w->nct * sub);
  w->hbt = off;
  off = align256(off + (size_t)bh * s->D * s->D * esz);
  w->hpart = off;
  off = align256(off + (size_t)bh * w->nch * s->D * s->D * sizeof(float));
  w->scores = off;  // only rows too long for k_route pass their scores through here
  if (n > pisa::kRouteMaxBlocks) off = align256(off + (size_t)route_chunk(bh, n) * n * n * sizeof(double));
  w->total = off;
  return PISA_OK;
}

pisa_status_t check_stats(const pisa_stats_t* st, const pisa::WsLayout& w, bool need_mnorm) {
  if (st == nullptr) return PISA_EINVAL;
  const double* p[] = {st->qbar, st->kbar, st->vsum, st->hbar};
  for (const double* x : p)
    if (x == nullptr || !aligned(x, 8)) return PISA_EINVAL;
  if (need_mnorm && st->mnorm == nullptr) return PISA_EINVAL;
  if (st->mnorm != nullptr && !aligned(st->mnorm, 8)) return PISA_EINVAL;
  if (st->mnorm_ord != PISA_NORM_FRO && st->mnorm_ord != PISA_NORM_SPECTRAL) return PISA_EINVAL;
  if (st->ws == nullptr || !aligned(st->ws, 256) || st->ws_bytes < w.total) return PISA_EINVAL;
  return PISA_OK;
}

bool tensor_ok(const void* p) { return p != nullptr && aligned(p, 16); }

pisa_status_t hip_status(hipError_t e) {
  if (e == hipSuccess) return PISA_OK;
  strncpy(g_last_hip_error, hipGetErrorString(e), sizeof(g_last_hip_error) - 1);
  g_last_hip_error[sizeof(g_last_hip_error) - 1] = '\0';
  return PISA_EHIP;
}

// Byte strides between batches, heads and tokens of a q, k, v or o tensor
// holding Lseg tokens of the sequence.
void io_strides(const pisa_shape_t* s, long Lseg, size_t* sb, size_t* sh, size_t* sl) {
  const size_t row = (size_t)s->D * (s->dtype == PISA_BF16 ? 2 : 4);
  *sb = row * s->H * Lseg;
  if (s->layout == PISA_LAYOUT_BLHD) {
    *sh = row;
    *sl = row * s->H;
  } else {
    *sh = row * Lseg;
    *sl = row;
  }
}

// Tokens in the first segment of the sequence (all of them without seg).
long seg_L0(const pisa_shape_t* s, const pisa_segments_t* seg) { return seg ? seg->L0 : s->L; }

// A second segment must hold 1 .. L-1 tokens and aligned tensors for what the
// call reads (and writes); L0 == L leaves it empty and its pointers unused.
pisa_status_t check_seg(const pisa_shape_t* s, const pisa_segments_t* seg, bool k_v, bool q_o) {
  if (seg == nullptr) return PISA_OK;
  if (seg->L0 < 1 || seg->L0 > s->L) return PISA_EINVAL;
  if (seg->L0 == s->L) return PISA_OK;
  if (!tensor_ok(seg->q1)) return PISA_EINVAL;
  if (k_v && (!tensor_ok(seg->k1) || !tensor_ok(seg->v1))) return PISA_EINVAL;
  if (q_o && !tensor_ok(seg->o1)) return PISA_EINVAL;
  return PISA_OK;
}

pisa::StatsArgs stats_args(const pisa_shape_t* s, const pisa::WsLayout& w, const void* q,
                           const void* k, const void* v, const pisa_segments_t* seg,
                           const pisa_stats_t* st, void* ws) {
  pisa::StatsArgs a;
  uint8_t* base = (uint8_t*)ws;
  a.q = (const uint8_t*)q;
  a.k = (const uint8_t*)k;
  a.v = (const uint8_t*)v;
  a.qbar = st ? st->qbar : nullptr;
  a.kbar = st ? st->kbar : nullptr;
  a.vsum = st ? st->vsum : nullptr;
  a.mnorm = st ? st->mnorm : nullptr;
  a.hbar = st ? st->hbar : nullptr;
  a.kp = base + w.kp;
  a.vp = base + w.vp;
  a.kbp = base + w.kbp;
  a.vbp = base + w.vbp;
  a.hbt = base + w.hbt;
  a.hpart = (float*)(base + w.hpart);
  a.kmax2 = (float*)(base + w.kmax2);
  const long L0 = seg_L0(s, seg);
  io_strides(s, L0, &a.stride_b, &a.stride_h, &a.stride_l);
  io_strides(s, s->L - L0, &a.stride1_b, &a.stride1_h, &a.stride1_l);
  a.q1 = (const uint8_t*)(seg ? seg->q1 : nullptr);
  a.k1 = (const uint8_t*)(seg ? seg->k1 : nullptr);
  a.v1 = (const uint8_t*)(seg ? seg->v1 : nullptr);
  a.L0 = (int)L0;
  a.H = s->H;
  a.L = s->L;
  a.n = w.n;
  a.blk = s->block;
  a.cb = w.cb;
  a.nch = w.nch;
  a.nct = w.nct;
  return a;
}

pisa::FwdArgs fwd_args(const pisa_shape_t* s, const pisa::WsLayout& w, const void* q, void* o,
                       const pisa_segments_t* seg, void* ws, const int32_t* idx, int topk,
                       double scale, int first_order, int tail) {
  pisa::FwdArgs a;
  uint8_t* base = (uint8_t*)ws;
  a.q = (const uint8_t*)q;
  a.o = (uint8_t*)o;
  a.kp = base + w.kp;
  a.vp = base + w.vp;
  a.kbp = base + w.kbp;
  a.vbp = base + w.vbp;
  a.hbt = base + w.hbt;
  a.idx = idx;
  a.kmax2 = (const float*)(base + w.kmax2);
  a.redo = (int*)(base + w.redo);
  a.sync = (int*)(base + w.sync);
  a.sync_ticks = 20000;  // 200 us, about one workgroup's lifetime at the Wan shape
  a.nch = w.nch;
  a.total = w.bh * w.n * w.spb;
  a.L = s->L;
  a.n = w.n;
  a.blk = s->block;
  a.topk = topk;
  a.n_last = s->L - (w.n - 1) * s->block;
  a.nct = w.nct;
  a.cs = (float)(scale * 1.4426950408889634);
  a.scale = (float)scale;
  a.first_order = first_order == 1;
  a.per_block = first_order == 2;
  a.tail = tail;
  const long L0 = seg_L0(s, seg);
  io_strides(s, L0, &a.stride_b, &a.stride_h, &a.stride_l);
  io_strides(s, s->L - L0, &a.stride1_b, &a.stride1_h, &a.stride1_l);
  a.q1 = (const uint8_t*)(seg ? seg->q1 : nullptr);
  a.o1 = (uint8_t*)(seg ? seg->o1 : nullptr);
  a.L0 = (int)L0;
  a.H = s->H;
  a.lse = nullptr;
  return a;
}

// Enqueues the statistics pass (arguments already validated).
pisa_status_t run_stats(const pisa_shape_t* shape, const pisa::WsLayout& w, const void* q,
                        const void* k, const void* v, const pisa_segments_t* seg,
                        const pisa_stats_t* st, hipStream_t s) {
  pisa_status_t rc;
  pisa::StatsArgs a = stats_args(shape, w, q, k, v, seg, st, st->ws);
  if ((rc = hip_status(pisa::launch_block_stats(shape->dtype, shape->D, pisa::kStatsFull, a, w.bh, s))))
    return rc;
  if ((rc = hip_status(pisa::launch_hbar_reduce(shape->dtype, shape->D, a, w.bh, s)))) return rc;
  if (st->mnorm == nullptr) return PISA_OK;
  if (st->mnorm_ord == PISA_NORM_SPECTRAL)
    return hip_status(pisa::launch_mnorm_spectral(shape->dtype, shape->D, a, w.bh, s));
  return hip_status(pisa::launch_block_stats(shape->dtype, shape->D, pisa::kStatsMnorm, a, w.bh, s));
}

// The checks pisa_attn_fwd and its variants share.
pisa_status_t check_fwd_args(const pisa::WsLayout& w, const void* q, const void* o,
                             int32_t first_order, const int32_t* idx, int32_t topk, double scale) {
  if (!tensor_ok(q) || !tensor_ok(o)) return PISA_EINVAL;
  if (!(scale > 0.0) || !isfinite(scale)) return PISA_EINVAL;
  if (first_order < 0 || first_order > 2) return PISA_EINVAL;
  if (topk < 1 || topk > w.n) return PISA_EINVAL;
  if (idx == nullptr || !aligned(idx, 4)) return PISA_EINVAL;
  return PISA_OK;
}

// ---- pisa_attn_fwd_noalloc: every intermediate in one fixed array per
// device. Host code never passes the array's own name to a kernel: its device
// address is looked up once per device and kept.
constexpr size_t kScratchBytes = PISA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint8_t* g_scratch_ptr[kMaxDevices] = {};

pisa_status_t scratch_on_current_device(uint8_t** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return PISA_ENOTSUP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    if (p == nullptr || !aligned(p, 256)) return PISA_EHIP;
    g_scratch_ptr[dev] = (uint8_t*)p;
  }
  *out = g_scratch_ptr[dev];
  return PISA_OK;
}

// Where the statistics sit in the scratch array: after the workspace regions
// the statistics pass and the fused pass use (the routing scores, the last
// region, are not needed).
struct NoAllocLayout {
  size_t qbar, kbar, vsum, hbar, total;
};

NoAllocLayout noalloc_layout(const pisa_shape_t* s, const pisa::WsLayout& w) {
  NoAllocLayout n;
  const size_t rows = (size_t)w.bh * w.n * s->D * sizeof(double);
  n.qbar = align256(w.scores);
  n.kbar = align256(n.qbar + rows);
  n.vsum = align256(n.kbar + rows);
  n.hbar = align256(n.vsum + rows);
  n.total = align256(n.hbar + (size_t)w.bh * s->D * s->D * sizeof(double));
  return n;
}

}  // namespace

PISA_API size_t pisa_workspace_bytes(const pisa_shape_t* shape) {
  pisa::WsLayout w;
  return check_shape(shape, &w) == PISA_OK ? w.total : 0;
}

PISA_API size_t dense_workspace_bytes(const pisa_shape_t* shape) {
  pisa::WsLayout w;
  return check_shape(shape, &w) == PISA_OK ? w.dense_total : 0;
}

PISA_API pisa_status_t pisa_block_stats_seg(const pisa_shape_t* shape, const void* q,
                                            const void* k, const void* v,
                                            const pisa_segments_t* seg, const pisa_stats_t* st,
                                            void* stream) {
  pisa::WsLayout w;
  pisa_status_t rc = check_shape(shape, &w);
  if (rc != PISA_OK) return rc;
  if (!tensor_ok(q) || !tensor_ok(k) || !tensor_ok(v)) return PISA_EINVAL;
  if ((rc = check_seg(shape, seg, true, false)) != PISA_OK) return rc;
  if ((rc = check_stats(st, w, false)) != PISA_OK) return rc;
  return run_stats(shape, w, q, k, v, seg, st, (hipStream_t)stream);
}

PISA_API pisa_status_t pisa_block_stats(const pisa_shape_t* shape, const void* q, const void* k,
                                        const void* v, const pisa_stats_t* st, void* stream) {
  return pisa_block_stats_seg(shape, q, k, v, nullptr, st, stream);
}

PISA_API pisa_status_t pisa_select(const pisa_shape_t* shape, const pisa_stats_t* st, double scale,
                                   double cov_weight, int32_t topk, int32_t sink_idx, int32_t* idx,
                                   void* stream) {
  pisa::WsLayout w;
  pisa_status_t rc = check_shape(shape, &w);
  if (rc != PISA_OK) return rc;
  if (!(scale > 0.0) || !isfinite(scale)) return PISA_EINVAL;
  if (!(cov_weight >= 0.0) || !isfinite(cov_weight)) return PISA_EINVAL;
  if (topk < 1 || topk > w.n) return PISA_EINVAL;
  if (sink_idx != PISA_SINK_NONE && sink_idx != 0 && sink_idx != -1) return PISA_EINVAL;
  if ((rc = check_stats(st, w, cov_weight > 0.0)) != PISA_OK) return rc;
  if (idx == nullptr || !aligned(idx, 4)) return PISA_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  if (w.n <= pisa::kRouteMaxBlocks) {
    pisa::RouteArgs ra;
    ra.qbar = st->qbar;
    ra.kbar = st->kbar;
    ra.mnorm = st->mnorm;
    ra.idx = idx;
    ra.scale = scale;
    ra.cov_weight = cov_weight;
    ra.n = w.n;
    ra.topk = topk;
    ra.sink_block = sink_idx == PISA_SINK_NONE ? -1 : (sink_idx == 0 ? 0 : w.n - 1);
    ra.nrt = (w.n + 15) / 16;
    ra.total = w.bh * ra.nrt;
    return hip_status(pisa::launch_route(shape->D, ra, s));
  }
  uint8_t* base = (uint8_t*)st->ws;
  pisa::ScoreArgs sa;
  sa.qbar = st->qbar;
  sa.kbar = st->kbar;
  sa.mnorm = st->mnorm;
  sa.scores = (double*)(base + w.scores);
  sa.scale = scale;
  sa.cov_weight = cov_weight;
  sa.n = w.n;
  sa.sink_block = sink_idx == PISA_SINK_NONE ? -1 : (sink_idx == 0 ? 0 : w.n - 1);
  pisa::TopkArgs ta;
  ta.scores = sa.scores;
  ta.n = w.n;
  ta.topk = topk;
  // heads in chunks that share one score buffer (stream order keeps them apart)
  const long chunk = route_chunk(w.bh, w.n);
  for (long h0 = 0; h0 < w.bh; h0 += chunk) {
    const long hc = w.bh - h0 < chunk ? w.bh - h0 : chunk;
    pisa::ScoreArgs sc = sa;
    sc.qbar = st->qbar + (size_t)h0 * w.n * shape->D;
    sc.kbar = st->kbar + (size_t)h0 * w.n * shape->D;
    sc.mnorm = st->mnorm ? st->mnorm + (size_t)h0 * w.n : nullptr;
    if (topk < w.n)
      if ((rc = hip_status(pisa::launch_scores(shape->D, sc, hc, s)))) return rc;
    ta.idx = idx + (size_t)h0 * w.n * topk;
    if ((rc = hip_status(pisa::launch_topk(ta, hc * w.n, s)))) return rc;
  }
  return PISA_OK;
}

PISA_API pisa_status_t pisa_attn_fwd_seg(const pisa_shape_t* shape, const void* q,
                                         const pisa_stats_t* st, int32_t first_order,
                                         const int32_t* idx, int32_t topk, double scale, void* o,
                                         const pisa_segments_t* seg, void* stream) {
  pisa::WsLayout w;
  pisa_status_t rc = check_shape(shape, &w);
  if (rc != PISA_OK) return rc;
  if ((rc = check_fwd_args(w, q, o, first_order, idx, topk, scale)) != PISA_OK) return rc;
  if ((rc = check_seg(shape, seg, false, true)) != PISA_OK) return rc;
  if ((rc = check_stats(st, w, false)) != PISA_OK) return rc;
  pisa::FwdArgs a = fwd_args(shape, w, q, o, seg, st->ws, idx, topk, scale, first_order, 1);
  return hip_status(pisa::launch_fwd(shape->dtype, shape->D, a, (hipStream_t)stream));
}

PISA_API pisa_status_t pisa_attn_fwd(const pisa_shape_t* shape, const void* q,
                                     const pisa_stats_t* st, int32_t first_order,
                                     const int32_t* idx, int32_t topk, double scale, void* o,
                                     void* stream) {
  return pisa_attn_fwd_seg(shape, q, st, first_order, idx, topk, scale, o, nullptr, stream);
}

PISA_API pisa_status_t pisa_attn_fwd_lse(const pisa_shape_t* shape, const void* q,
                                         const pisa_stats_t* st, int32_t first_order,
                                         const int32_t* idx, int32_t topk, double scale, void* o,
                                         float* lse, void* stream) {
  pisa::WsLayout w;
  pisa_status_t rc = check_shape(shape, &w);
  if (rc != PISA_OK) return rc;
  if ((rc = check_fwd_args(w, q, o, first_order, idx, topk, scale)) != PISA_OK) return rc;
  if (lse == nullptr || !aligned(lse, 4)) return PISA_EINVAL;
  if ((rc = check_stats(st, w, false)) != PISA_OK) return rc;
  pisa::FwdArgs a = fwd_args(shape, w, q, o, nullptr, st->ws, idx, topk, scale, first_order, 1);
  a.lse = lse;
  return hip_status(pisa::launch_fwd(shape->dtype, shape->D, a, (hipStream_t)stream));
}

PISA_API pisa_status_t pisa_attn_fwd_noalloc(const pisa_shape_t* shape, const void* q,
                                             const void* k, const void* v, int32_t first_order,
                                             const int32_t* idx, int32_t topk, double scale,
                                             void* o, void* stream) {
  pisa::WsLayout w;
  pisa_status_t rc = check_shape(shape, &w);
  if (rc != PISA_OK) return rc;
  if (!tensor_ok(k) || !tensor_ok(v)) return PISA_EINVAL;
  if ((rc = check_fwd_args(w, q, o, first_order, idx, topk, scale)) != PISA_OK) return rc;
  const NoAllocLayout nl = noalloc_layout(shape, w);
  if (nl.total > kScratchBytes) return PISA_ETOOBIG;
  uint8_t* base = nullptr;
  if ((rc = scratch_on_current_device(&base)) != PISA_OK) return rc;
  pisa_stats_t st;
  st.qbar = (double*)(base + nl.qbar);
  st.kbar = (double*)(base + nl.kbar);
  st.vsum = (double*)(base + nl.vsum);
  st.hbar = (double*)(base + nl.hbar);
  st.mnorm = nullptr;
  st.mnorm_ord = PISA_NORM_FRO;
  st.ws = base;
  st.ws_bytes = nl.total;
  hipStream_t s = (hipStream_t)stream;
  if ((rc = run_stats(shape, w, q, k, v, nullptr, &st, s)) != PISA_OK) return rc;
  pisa::FwdArgs a = fwd_args(shape, w, q, o, nullptr, base, idx, topk, scale, first_order, 1);
  return hip_status(pisa::launch_fwd(shape->dtype, shape->D, a, s));
}

namespace {

pisa::BwdLayout bwd_layout(const pisa_shape_t* s, const pisa::WsLayout& w) {
  pisa::BwdLayout b;
  const int W = (w.n + 31) / 32;
  size_t off = 0;
  b.selmap = off;
  off = align256(off + (size_t)w.bh * w.n * W * sizeof(uint32_t));
  b.lse = off;
  off = align256(off + (size_t)w.bh * w.n * s->block * sizeof(float));
  b.delta = off;
  off = align256(off + (size_t)w.bh * w.n * s->block * sizeof(float));
  b.dkbar = off;
  off = align256(off + (size_t)w.bh * w.n * s->D * sizeof(float));
  b.dvsum = off;
  off = align256(off + (size_t)w.bh * w.n * s->D * sizeof(float));
  b.kbt = off;
  off = align256(off + (size_t)w.bh * w.nct * 64 * s->D * w.esz);
  b.vbt = off;
  off = align256(off + (size_t)w.bh * w.nct * 64 * s->D * w.esz);
  // The centroid gradients take one workgroup per (head, tile of 64
  // centroids) and range of query blocks: enough ranges for about 1024
  // workgroups, each of at least 8 query blocks, at most 16.
  const long tiles = w.bh * w.nct;
  long parts = (1024 + tiles - 1) / tiles;
  parts = parts > 16 ? 16 : parts;
  parts = parts > w.n / 8 ? w.n / 8 : parts;
  b.cparts = parts < 1 ? 1 : (int)parts;
  const size_t pbytes = b.cparts > 1 ? (size_t)b.cparts * w.bh * w.nct * 64 * s->D * sizeof(float) : 0;
  b.dkbar_p = off;
  off = align256(off + pbytes);
  b.dvsum_p = off;
  off = align256(off + pbytes);
  b.sync = off;
  off = align256(off + sizeof(int32_t));
  b.total = off;
  return b;
}

}  // namespace

PISA_API size_t pisa_bwd_workspace_bytes(const pisa_shape_t* shape) {
  pisa::WsLayout w;
  return check_shape(shape, &w) == PISA_OK ? bwd_layout(shape, w).total : 0;
}

PISA_API pisa_status_t pisa_attn_bwd(const pisa_shape_t* shape, const void* q, const void* k,
                                     const void* v, const pisa_stats_t* st, const int32_t* idx,
                                     int32_t topk, double scale, const void* o, const float* lse,
                                     const void* dout, void* dq, void* dk, void* dv, void* ws,
                                     size_t ws_bytes, void* stream) {
  pisa::WsLayout w;
  pisa_status_t rc = check_shape(shape, &w);
  if (rc != PISA_OK) return rc;
  const void* in[] = {q, k, v, o, dout, dq, dk, dv};
  for (const void* p : in)
    if (!tensor_ok(p)) return PISA_EINVAL;
  if (!(scale > 0.0) || !isfinite(scale)) return PISA_EINVAL;
  if (topk < 1 || topk > w.n) return PISA_EINVAL;
  if (idx == nullptr || !aligned(idx, 4)) return PISA_EINVAL;
  if (lse != nullptr && !aligned(lse, 4)) return PISA_EINVAL;
  if (st == nullptr || st->kbar == nullptr || st->vsum == nullptr || !aligned(st->kbar, 8) ||
      !aligned(st->vsum, 8))
    return PISA_EINVAL;
  const pisa::BwdLayout bl = bwd_layout(shape, w);
  if (ws == nullptr || !aligned(ws, 256) || ws_bytes < bl.total) return PISA_EINVAL;
  uint8_t* base = (uint8_t*)ws;
  pisa::BwdArgs a;
  a.q = (const uint8_t*)q;
  a.k = (const uint8_t*)k;
  a.v = (const uint8_t*)v;
  a.o = (const uint8_t*)o;
  a.dout = (const uint8_t*)dout;
  a.dq = (uint8_t*)dq;
  a.dk = (uint8_t*)dk;
  a.dv = (uint8_t*)dv;
  io_strides(shape, shape->L, &a.stride_b, &a.stride_h, &a.stride_l);
  a.H = shape->H;
  a.kbar = st->kbar;
  a.vsum = st->vsum;
  a.idx = idx;
  a.selmap = (uint32_t*)(base + bl.selmap);
  a.lse = (float*)(base + bl.lse);
  a.lse_in = lse;
  a.delta = (float*)(base + bl.delta);
  a.dkbar = (float*)(base + bl.dkbar);
  a.dvsum = (float*)(base + bl.dvsum);
  a.kbt = base + bl.kbt;
  a.vbt = base + bl.vbt;
  a.cparts = bl.cparts;
  a.dkbar_p = (float*)(base + bl.dkbar_p);
  a.dvsum_p = (float*)(base + bl.dvsum_p);
  a.L = shape->L;
  a.n = w.n;
  a.blk = shape->block;
  a.n_last = shape->L - (w.n - 1) * shape->block;
  a.nct = w.nct;
  a.topk = topk;
  a.W = (w.n + 31) / 32;
  a.scale = (float)scale;
  a.sync = (int*)(base + bl.sync);
  a.sync_ticks = 50000;  // 500 us, about one query tile's lifetime in k_bwd_dq at the Wan shape
  a.total = w.bh * w.n * (shape->block / 64);
  return hip_status(pisa::launch_bwd(shape->dtype, shape->D, a, w.bh, (hipStream_t)stream));
}

PISA_API pisa_status_t dense_attn_fwd_seg(const pisa_shape_t* shape, const void* q, const void* k,
                                          const void* v, const pisa_segments_t* seg, double scale,
                                          void* o, void* ws, size_t ws_bytes, void* stream) {
  pisa::WsLayout w;
  pisa_status_t rc = check_shape(shape, &w);
  if (rc != PISA_OK) return rc;
  if (!tensor_ok(q) || !tensor_ok(k) || !tensor_ok(v) || !tensor_ok(o)) return PISA_EINVAL;
  if ((rc = check_seg(shape, seg, true, true)) != PISA_OK) return rc;
  if (!(scale > 0.0) || !isfinite(scale)) return PISA_EINVAL;
  if (ws == nullptr || !aligned(ws, 256) || ws_bytes < w.dense_total) return PISA_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  pisa::StatsArgs sa = stats_args(shape, w, q, k, v, seg, nullptr, ws);
  if ((rc = hip_status(pisa::launch_block_stats(shape->dtype, shape->D, pisa::kStatsPackOnly, sa, w.bh, s))))
    return rc;
  pisa::FwdArgs a = fwd_args(shape, w, q, o, seg, ws, nullptr, w.n, scale, 0, 0);
  return hip_status(pisa::launch_fwd(shape->dtype, shape->D, a, s));
}

PISA_API pisa_status_t dense_attn_fwd(const pisa_shape_t* shape, const void* q, const void* k,
                                      const void* v, double scale, void* o, void* ws,
                                      size_t ws_bytes, void* stream) {
  return dense_attn_fwd_seg(shape, q, k, v, nullptr, scale, o, ws, ws_bytes, stream);
}

PISA_API const char* pisa_status_string(pisa_status_t status) {
  switch (status) {
    case PISA_OK: return "ok";
    case PISA_EINVAL: return "invalid argument";
    case PISA_ENOTSUP: return "unsupported shape or dtype";
    case PISA_EHIP: return "HIP runtime error";
    case PISA_ETOOBIG: return "problem larger than the fixed scratch of pisa_attn_fwd_noalloc";
  }
  return "unknown status";
}

PISA_API const char* pisa_last_hip_error(void) { return g_last_hip_error; }
