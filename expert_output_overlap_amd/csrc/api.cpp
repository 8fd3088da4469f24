// C ABI of the MoE expert-compute-plus-return path (declarations and contracts in include/moe_overlap.h).
// Host side only: argument checks, workspace carving, launches on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/moe_overlap.h"
#include "common.h"
#include "item_list.h"
#include "launch.h"

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

// Returns "" when the shape is valid.
std::string check_shape(const moe_shape* s) {
  if (s == nullptr) return "null shape";
  if (s->R < 1 || s->R > MOE_MAX_OWNERS) return "R must be in [1, 16]";
  if (s->tokens_per_owner < 0) return "tokens_per_owner must be >= 0";
  if (s->num_local_experts < 1 || s->num_local_experts > MOE_MAX_LOCAL_EXPERTS) return "num_local_experts in [1, 64]";
  if (s->num_global_experts < 1 || s->num_global_experts > 1024) return "num_global_experts in [1, 1024]";
  if (s->num_global_experts % s->num_local_experts) return "num_global_experts % num_local_experts != 0";
  if (s->top_k < 1 || s->top_k > 16 || s->top_k > s->num_global_experts) return "top_k in [1, min(G, 16)]";
  if (s->self_rank < 0 || s->self_rank >= s->R ||
      (int64_t)(s->self_rank + 1) * s->num_local_experts > s->num_global_experts)
    return "self_rank out of range";
  if (s->d < 64 || s->d % 64) return "d must be a positive multiple of 64";
  if (s->f < 64 || s->f % 64) return "f must be a positive multiple of 64";
  if (s->tile_m < 16 || s->tile_m > 256 || s->tile_m % 16) return "tile_m must be a multiple of 16 in [16, 256]";
  if (s->seg_bands < 1) return "seg_bands must be >= 1";
  if (s->dtype != MOE_BF16 && s->dtype != MOE_F32) return "dtype must be MOE_BF16 or MOE_F32";
  const int64_t T = (int64_t)s->R * s->tokens_per_owner;
  if (T * s->top_k >= (1ll << 31)) return "T*k too large";
  const int64_t cap = (T * std::min(s->top_k, s->num_local_experts) +
                       (int64_t)s->num_local_experts * s->R * (s->tile_m - 1));
  if (cap >= (1ll << 30)) return "padded row capacity too large";
  // the GEMMs address rows of x_pad / h and of one expert's weights with 32-bit byte offsets
  const int64_t esize = s->dtype == MOE_BF16 ? 2 : 4;
  const int64_t kmax = s->d > s->f ? s->d : s->f;
  if ((cap + 256) * kmax * esize >= (1ll << 32) || 2ll * s->f * s->d * esize >= (1ll << 32))
    return "rows x width too large for 32-bit offsets";
  return "";
}

int64_t capacity_rows(const moe_shape* s) {
  const int64_t T = (int64_t)s->R * s->tokens_per_owner;
  const int64_t bound = T * std::min(s->top_k, s->num_local_experts) +
                        (int64_t)s->num_local_experts * s->R * (s->tile_m - 1);
  return round_up(bound, s->tile_m);
}

struct Carve {
  int64_t off = 0;
  int64_t take(int64_t elems, int64_t esize) {
    const int64_t o = off;
    off = round_up(off + elems * esize, 256);
    return o;
  }
};

struct Offsets {
  int64_t counts, padded_off, recv_off, tile_owner, tile_expert, tile_valid, tile_order, seg_desc, row_src,
      combine_plan, scalars, status, mtile_desc, seg_mtiles, seg_sched, chunk_counts, mt_order, total;
  int64_t cap_rows, cap_tiles, cap_mtiles;
};

Offsets layout_offsets(const moe_shape* s) {
  Offsets o;
  const int64_t NG = (int64_t)s->num_local_experts * s->R;
  const int64_t T = (int64_t)s->R * s->tokens_per_owner;
  o.cap_rows = capacity_rows(s);
  o.cap_tiles = o.cap_rows / s->tile_m;
  const int mt_rows = ffn_gemm_bm(s->dtype);
  o.cap_mtiles = (o.cap_rows + mt_rows - 1) / mt_rows + NG + 1;
  const int64_t n_chunks = (s->tokens_per_owner + 63) / 64;
  Carve c;
  o.counts = c.take(NG, 4);
  o.padded_off = c.take(NG, 4);
  o.recv_off = c.take(NG, 4);
  o.tile_owner = c.take(o.cap_tiles, 4);
  o.tile_expert = c.take(o.cap_tiles, 4);
  o.tile_valid = c.take(o.cap_tiles, 4);
  o.tile_order = c.take(o.cap_tiles, 4);
  o.seg_desc = c.take(o.cap_tiles * MOE_SEG_FIELDS, 4);
  o.row_src = c.take(o.cap_rows, 4);
  o.combine_plan = c.take(T * s->top_k, 4);
  o.scalars = c.take(5 + s->R, 4);
  o.status = c.take(1, 4);
  o.mtile_desc = c.take(o.cap_mtiles * MOE_MT_FIELDS, 4);
  o.seg_mtiles = c.take(o.cap_tiles * 2, 4);
  o.seg_sched = c.take(o.cap_tiles, 4);
  o.chunk_counts = c.take((int64_t)s->R * n_chunks * s->num_local_experts, 4);
  o.mt_order = c.take(o.cap_mtiles, 4);
  o.total = c.off;
  return o;
}

std::mutex g_mu;

int device_cus(int dev) {
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  return n;
}

// Optional kernel timing: per call, a start and an end event for each launch the call makes, taken by the
// launch itself (hipExtLaunchKernel), so timing puts no marker in the stream.  Pair 0 is the producer launch,
// then the fp32 second GEMM if there is one, then the sequential-mode consumer if there is one.
struct CallEvents {
  hipEvent_t e[6];
  int n = 0;            // launches timed (pairs used)
  bool second = false;  // pair 1 is the fp32 second GEMM
  bool cons = false;    // the last pair is the sequential-mode consumer
  void destroy() {
    for (int i = 0; i < 6; ++i) hipEventDestroy(e[i]);
  }
};
bool g_timing = false;
std::vector<CallEvents> g_events;

int timing_begin(CallEvents* ce) {
  for (int i = 0; i < 6; ++i)
    if (hipEventCreate(&ce->e[i]) != hipSuccess) {
      for (int j = 0; j < i; ++j) hipEventDestroy(ce->e[j]);
      return -1;
    }
  return 0;
}

}  // namespace

extern "C" {

int moe_set_kernel_timing(int enable) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_timing = enable != 0;
  return MOE_OK;
}

int moe_kernel_times(double* out4) {
  if (!out4) return fail(MOE_EINVAL, "null pointer");
  std::lock_guard<std::mutex> lk(g_mu);
  double t[3] = {0, 0, 0};
  int rc = MOE_OK;
  for (auto& ce : g_events) {
    float ms = 0;
    for (int i = 0; i < 2 * ce.n; ++i)
      if (hipEventSynchronize(ce.e[i]) != hipSuccess) rc = MOE_EHIP;
    auto pair = [&](int j, double* acc) {
      if (hipEventElapsedTime(&ms, ce.e[2 * j], ce.e[2 * j + 1]) == hipSuccess) *acc += ms;
      else rc = MOE_EHIP;
    };
    if (ce.n > 0) pair(0, &t[0]);
    if (ce.second) pair(1, &t[1]);
    if (ce.cons) pair(ce.n - 1, &t[2]);
    ce.destroy();
  }
  out4[0] = t[0];
  out4[1] = t[1];
  out4[2] = t[2];
  out4[3] = (double)g_events.size();
  g_events.clear();
  if (rc != MOE_OK) return fail(rc, "event timing failed");
  return MOE_OK;
}

const char* moe_last_error(void) { return g_err.c_str(); }

const char* moe_version(void) { return "moe_overlap gfx950 1"; }

int moe_route(const moe_shape* s, const float* logits, int32_t* topk_idx, float* topk_w, void* stream) {
  const std::string e = check_shape(s);
  if (!e.empty()) return fail(MOE_EINVAL, e);
  const int64_t T = (int64_t)s->R * s->tokens_per_owner;
  if (T > 0 && (!logits || !topk_idx || !topk_w)) return fail(MOE_EINVAL, "null pointer");
  if (launch_route((int)T, s->num_global_experts, s->top_k, logits, topk_idx, topk_w, (hipStream_t)stream))
    return fail(MOE_EHIP, "route launch failed");
  return MOE_OK;
}

int64_t moe_layout_capacity_rows(const moe_shape* s) {
  if (!check_shape(s).empty()) return -1;
  return capacity_rows(s);
}

int64_t moe_layout_workspace_bytes(const moe_shape* s) {
  if (!check_shape(s).empty()) return -1;
  return layout_offsets(s).total;
}

int moe_layout_bind(const moe_shape* s, void* workspace, int64_t workspace_bytes, moe_layout* L) {
  const std::string e = check_shape(s);
  if (!e.empty()) return fail(MOE_EINVAL, e);
  if (!workspace || !L) return fail(MOE_EINVAL, "null pointer");
  if (((uintptr_t)workspace) % 256) return fail(MOE_EINVAL, "workspace must be 256-byte aligned");
  const Offsets o = layout_offsets(s);
  if (workspace_bytes < o.total) return fail(MOE_EINVAL, "workspace too small");
  char* b = (char*)workspace;
  L->counts = (int32_t*)(b + o.counts);
  L->padded_off = (int32_t*)(b + o.padded_off);
  L->recv_off = (int32_t*)(b + o.recv_off);
  L->tile_owner = (int32_t*)(b + o.tile_owner);
  L->tile_expert = (int32_t*)(b + o.tile_expert);
  L->tile_valid = (int32_t*)(b + o.tile_valid);
  L->tile_order = (int32_t*)(b + o.tile_order);
  L->seg_desc = (int32_t*)(b + o.seg_desc);
  L->row_src = (int32_t*)(b + o.row_src);
  L->combine_plan = (int32_t*)(b + o.combine_plan);
  L->scalars = (int32_t*)(b + o.scalars);
  L->status = (int32_t*)(b + o.status);
  L->mtile_desc = (int32_t*)(b + o.mtile_desc);
  L->seg_mtiles = (int32_t*)(b + o.seg_mtiles);
  L->seg_sched = (int32_t*)(b + o.seg_sched);
  L->chunk_counts = (int32_t*)(b + o.chunk_counts);
  L->mt_order = (int32_t*)(b + o.mt_order);
  L->cap_rows = o.cap_rows;
  L->cap_tiles = o.cap_tiles;
  L->cap_mtiles = o.cap_mtiles;
  return MOE_OK;
}

static bool layout_ok(const moe_layout* L) {
  return L && L->counts && L->padded_off && L->recv_off && L->tile_owner && L->tile_expert && L->tile_valid &&
         L->tile_order && L->seg_desc && L->row_src && L->combine_plan && L->scalars && L->status &&
         L->mtile_desc && L->seg_mtiles && L->seg_sched && L->chunk_counts && L->mt_order && L->cap_rows > 0;
}

int moe_layout_build(const moe_shape* s, const int32_t* topk_idx, const void* x, moe_layout* L, void* x_pad,
                     void* stream) {
  const std::string e = check_shape(s);
  if (!e.empty()) return fail(MOE_EINVAL, e);
  if (!layout_ok(L)) return fail(MOE_EINVAL, "layout not bound");
  const int64_t T = (int64_t)s->R * s->tokens_per_owner;
  if (T > 0 && (!topk_idx || (x && !x_pad))) return fail(MOE_EINVAL, "null pointer");
  if (L->cap_tiles * s->tile_m != L->cap_rows) return fail(MOE_EINVAL, "layout bound for another tile_m");
  LayoutLaunch p;
  p.topk_idx = topk_idx;
  p.x = x;
  p.x_pad = x_pad;
  p.L = L;
  p.R = s->R;
  p.T_o = s->tokens_per_owner;
  p.G = s->num_global_experts;
  p.k = s->top_k;
  p.lo = s->self_rank * s->num_local_experts;
  p.E = s->num_local_experts;
  p.M = s->tile_m;
  p.mgb = s->seg_bands;
  p.self_rank = s->self_rank;
  p.mt_rows = ffn_gemm_bm(s->dtype);
  p.row_bytes = (int64_t)s->d * (s->dtype == MOE_BF16 ? 2 : 4);
  if (launch_layout(p, (hipStream_t)stream)) return fail(MOE_EHIP, "layout launch failed");
  return MOE_OK;
}

int moe_read_status(const moe_layout* L, void* stream) {
  if (!L || !L->status) return fail(MOE_EINVAL, "null layout");
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return fail(MOE_EHIP, "stream sync failed");
  int32_t v = 0;
  if (hipMemcpy(&v, L->status, 4, hipMemcpyDeviceToHost) != hipSuccess) return fail(MOE_EHIP, "status copy failed");
  return v;
}

int64_t moe_ffn_flags_count(const moe_shape* s) {
  if (!check_shape(s).empty()) return -1;
  const Offsets o = layout_offsets(s);
  return ffn_flag_words(s->dtype, s->d, s->f, o.cap_mtiles);
}

int32_t moe_pick_consumer_cus(const moe_shape* s, int32_t n_cu) {
  if (!check_shape(s).empty() || n_cu < 2) return -1;
  if (s->dtype != MOE_BF16) return std::min(8, std::max(1, std::min(32, n_cu / 4)));
  // the launch's own rule (ffn_adaptive_consumers) before any observation, with the rows of R - 1 of the R owners
  // returned (uniform routing), in full row tiles
  const int64_t m = 1000000;
  int n1 = 0, n2 = 0, S = 0;
  ffn_list_dims(s->d, s->f, &n1, &n2, &S);
  return ffn_adaptive_consumers(n_cu, m, m * (s->R - 1) / s->R, s->d, s->f, (m + 255) / 256 * n1, 0.f, 0.f);
}

int32_t moe_pick_consumer_cus_observed(const moe_shape* s, int32_t n_cu, int64_t rows_routed, int64_t rows_returned,
                                       int32_t n_mtiles, float ffn_rate, float copy_rate) {
  if (!check_shape(s).empty() || n_cu < 2 || rows_routed < 0 || rows_returned < 0 || rows_returned > rows_routed ||
      n_mtiles < 0)
    return -1;
  if (s->dtype != MOE_BF16) return moe_pick_consumer_cus(s, n_cu);
  int n1 = 0, n2 = 0, S = 0;
  ffn_list_dims(s->d, s->f, &n1, &n2, &S);
  return ffn_adaptive_consumers(n_cu, rows_routed, rows_returned, s->d, s->f, (int64_t)n_mtiles * n1, ffn_rate,
                                copy_rate);
}

}  // extern "C"

namespace {
// Mode 3: the return on the DMA engines (review page of FiCCO, "If this is right": DMA-offloaded transfers contend
// less with the GEMMs than copies on the compute units).  The FFN's item list runs as a few launches, cut at GEMM2
// window boundaries (a y tile's k-splits never straddle two launches); after each launch an event gates the copy
// streams that move the segments the launch completed with hipMemcpyDeviceToDeviceNoCU copies (DMA engines, no
// CUs) while the next launch computes.  One DMA engine copies HBM to HBM at ~50 GB/s (measured), so the copies
// are spread over DMA_STREAMS streams, each to the one with the fewest bytes queued.  The host needs the segment table for the copies: it reads it back after
// synchronising the caller's stream (the layout build), once per call.
#define DMA_STREAMS 3  // copy streams: with the caller's stream, the four hardware queues of a process
struct DmaCtx {
  hipStream_t copy[DMA_STREAMS] = {};
  hipEvent_t ev[4] = {};            // end of each launch chunk, on the caller's stream
  hipEvent_t done[DMA_STREAMS] = {};  // end of each copy stream's work
};
std::vector<DmaCtx> g_dma;  // per device, guarded by g_mu

int ffn_dma(const moe_shape* s, const moe_layout* L, FfnLaunch& p, int n_cu, int dev, hipStream_t st, CallEvents* ce,
            bool timed) {
  DmaCtx* ctx;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    if ((int)g_dma.size() <= dev) g_dma.resize(dev + 1);
    ctx = &g_dma[dev];
    if (ctx->copy[DMA_STREAMS - 1] == nullptr) {
      for (auto& c : ctx->copy)
        if (c == nullptr && hipStreamCreateWithFlags(&c, hipStreamNonBlocking) != hipSuccess) {
          c = nullptr;
          return fail(MOE_EHIP, "copy stream creation failed");
        }
      for (auto& e : ctx->ev)
        if (e == nullptr && hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) {
          e = nullptr;
          return fail(MOE_EHIP, "event creation failed");
        }
      for (auto& e : ctx->done)
        if (e == nullptr && hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) {
          e = nullptr;
          return fail(MOE_EHIP, "event creation failed");
        }
    }
  }
  // the segment table and the producer's row-tile order, on the host
  const int R = s->R;
  if (hipStreamSynchronize(st) != hipSuccess) return fail(MOE_EHIP, "stream sync failed");
  std::vector<int32_t> sc(5 + R);
  int32_t status = 0;
  if (hipMemcpy(&status, L->status, 4, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(sc.data(), L->scalars, sc.size() * 4, hipMemcpyDeviceToHost) != hipSuccess)
    return fail(MOE_EHIP, "layout readback failed");
  if (status != MOE_OK) return MOE_OK;  // the device status already reports the failure; nothing runs after it
  const int n_segs = sc[SC_NSEGS], n_mt = sc[SC_NR + R], n_rem = sc[SC_NR + R + 1];
  if (n_mt == 0) return MOE_OK;
  std::vector<int32_t> seg(8 * (size_t)n_segs), segm(2 * (size_t)n_segs), order(n_mt);
  if ((n_segs > 0 && (hipMemcpy(seg.data(), L->seg_desc, seg.size() * 4, hipMemcpyDeviceToHost) != hipSuccess ||
                      hipMemcpy(segm.data(), L->seg_mtiles, segm.size() * 4, hipMemcpyDeviceToHost) != hipSuccess)) ||
      hipMemcpy(order.data(), L->mt_order, order.size() * 4, hipMemcpyDeviceToHost) != hipSuccess)
    return fail(MOE_EHIP, "layout readback failed");
  // the list (GEMM1 first, no half-width round, no consumer workgroups) and its chunks: windows of the GEMM2 part
  int n1, n2, S;
  ffn_list_dims(s->d, s->f, &n1, &n2, &S);
  const int W = p.band_window > 0 ? p.band_window : 4;
  const FfnList Lst = ffn_list_make(n_mt, p.tile_order == 0 ? n_rem : n_mt, n1, n2, S, W, 0, 0, n_cu, false);
  const int64_t g1 = (int64_t)n_mt * n1;
  const int nw = (n_mt + W - 1) / W, K = std::min(4, nw);
  auto wstart = [&](int w) { return g1 + (int64_t)std::min(w * W, n_mt) * n2 * S; };
  std::vector<int64_t> cb(K + 1);
  cb[0] = 0;
  for (int c = 1; c <= K; ++c) cb[c] = wstart((int)((int64_t)c * nw / K));
  // the chunk that completes each row tile (its last second-GEMM item), then each segment
  std::vector<int> done(n_mt, 0);
  for (int c = 0; c < K; ++c)
    for (int64_t i = std::max(cb[c], g1); i < cb[c + 1]; ++i) {
      const FfnSlot sl = ffn_slot((int)i, Lst);
      const int mt = p.tile_order == 0 ? order[sl.pos] : sl.pos;
      done[mt] = std::max(done[mt], c);
    }
  const int64_t row_bytes = (int64_t)s->d * 2;
  const char* y = (const char*)p.y_pad;
  int64_t queued[DMA_STREAMS] = {};  // bytes given to each copy stream: each copy goes to the least loaded
  for (int c = 0; c < K; ++c) {
    p.item_begin = (int)cb[c];
    p.item_end = (int)cb[c + 1];
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (timed && c == 0) e0 = ce->e[0];
    if (timed && c == K - 1) e1 = ce->e[1];
    if (launch_ffn_producer(p, n_cu, 0, st, e0, e1)) return fail(MOE_EHIP, "producer launch failed");
    if (hipEventRecord(ctx->ev[c], st) != hipSuccess) return fail(MOE_EHIP, "event failed");
    for (auto cs : ctx->copy)
      if (hipStreamWaitEvent(cs, ctx->ev[c], 0) != hipSuccess) return fail(MOE_EHIP, "event failed");
    // the segments this chunk completed, other owners only, contiguous runs of one owner merged into one copy
    std::vector<int> mine;
    for (int i = 0; i < n_segs; ++i) {
      const int32_t* sd = &seg[8 * (size_t)i];
      if (sd[SEG_OWNER] == s->self_rank || sd[SEG_ROWS] == 0) continue;
      int c_seg = 0;
      for (int m = segm[2 * i]; m < segm[2 * i] + segm[2 * i + 1]; ++m) c_seg = std::max(c_seg, done[m]);
      if (c_seg == c) mine.push_back(i);
    }
    std::sort(mine.begin(), mine.end(), [&](int a, int b) {
      const int32_t *x = &seg[8 * (size_t)a], *z = &seg[8 * (size_t)b];
      return x[SEG_OWNER] != z[SEG_OWNER] ? x[SEG_OWNER] < z[SEG_OWNER] : x[SEG_DST_ROW] < z[SEG_DST_ROW];
    });
    for (size_t k = 0; k < mine.size();) {
      const int32_t* sd = &seg[8 * (size_t)mine[k]];
      const int owner = sd[SEG_OWNER];
      int64_t src = sd[SEG_SRC_ROW], dst = sd[SEG_DST_ROW], rows = sd[SEG_ROWS];
      size_t j = k + 1;
      for (; j < mine.size(); ++j) {
        const int32_t* nx = &seg[8 * (size_t)mine[j]];
        if (nx[SEG_OWNER] != owner || nx[SEG_SRC_ROW] != src + rows || nx[SEG_DST_ROW] != dst + rows) break;
        rows += nx[SEG_ROWS];
      }
      const int q = (int)(std::min_element(queued, queued + DMA_STREAMS) - queued);
      queued[q] += rows * row_bytes;
      if (hipMemcpyAsync((char*)p.recv[owner] + dst * row_bytes, y + src * row_bytes, rows * row_bytes,
                         hipMemcpyDeviceToDeviceNoCU, ctx->copy[q]) != hipSuccess)
        return fail(MOE_EHIP, "DMA copy failed");
      k = j;
    }
  }
  for (int q = 0; q < DMA_STREAMS; ++q)
    if (hipEventRecord(ctx->done[q], ctx->copy[q]) != hipSuccess || hipStreamWaitEvent(st, ctx->done[q], 0) != hipSuccess)
      return fail(MOE_EHIP, "event failed");
  return MOE_OK;
}

// The body of moe_expert_ffn_overlap; flags == nullptr selects the allocation-free variant's own flag buffer.
int ffn_overlap(const moe_shape* s, const moe_layout* L, const void* x_pad, const void* w_gate_up, const void* w_down,
                void* h_ws, void* y_pad, void* const* recv, uint32_t* flags, const moe_overlap_cfg* cfg_in,
                void* stream) {
  const std::string e = check_shape(s);
  if (!e.empty()) return fail(MOE_EINVAL, e);
  if (!layout_ok(L) || !cfg_in) return fail(MOE_EINVAL, "null layout or cfg");
  if (!x_pad || !w_gate_up || !w_down || !h_ws || !y_pad || !recv)
    return fail(MOE_EINVAL, "null pointer");
  moe_overlap_cfg cfg_v = *cfg_in;
  const moe_overlap_cfg* cfg = &cfg_v;
  for (int r = 0; r < s->R; ++r)
    if (!recv[r]) return fail(MOE_EINVAL, "null receive buffer");
  if ((uintptr_t)flags % 8 != 0) return fail(MOE_EINVAL, "flags must be 8-byte aligned");
  if (cfg->epoch == 0 && flags != nullptr) return fail(MOE_EINVAL, "epoch must be nonzero");
  if (cfg->mode < 0 || cfg->mode > 3) return fail(MOE_EINVAL, "mode must be 0, 1, 2 or 3");
  if (cfg->mode == 3 && (s->dtype != MOE_BF16 || flags == nullptr))
    return fail(MOE_EINVAL, "mode 3 (return on the DMA engines) is for bf16 with a flag workspace");
  if (cfg->band_window < 0) return fail(MOE_EINVAL, "band_window must be >= 0");
  if (cfg->tile_order != 0 && cfg->tile_order != 1) return fail(MOE_EINVAL, "tile_order must be 0 or 1");
  if (cfg->x_tokens && (s->dtype != MOE_BF16 || (cfg->mode != 0 && cfg->mode != 1)))
    return fail(MOE_EINVAL, "x_tokens (rows landed by the launch) is for bf16 in mode 0 or 1");
  if (cfg->gu_out && (s->dtype != MOE_BF16 || cfg->mode == 2 || s->f % 128))
    return fail(MOE_EINVAL, "gu_out (the first GEMM's pre-activations, for the backward) is for bf16 shapes with f a "
                            "multiple of 128, in mode 0, 1 or 3");
  hipStream_t st = (hipStream_t)stream;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(MOE_EHIP, "hipGetDevice failed");
  const int n_cu = device_cus(dev);
  if (n_cu <= 0) return fail(MOE_EHIP, "cannot query the CU count");
  if (cfg->consumer_cus < -1 || cfg->consumer_cus > n_cu / 2)
    return fail(MOE_EINVAL, "consumer_cus must be -1 (none), 0 (library pick) or in [1, CUs/2]");
  if (cfg->consumer_cus == -1 && (s->dtype != MOE_BF16 || (cfg->mode != 0 && cfg->mode != 1)))
    return fail(MOE_EINVAL, "consumer_cus = -1 (no consumer partition) is for bf16 in mode 0 or 1");
  // a partition for the launches that need one: the return alone (mode 2), fp32, a fixed bf16 choice
  const int C = cfg->consumer_cus > 0 ? cfg->consumer_cus : std::max(1, moe_pick_consumer_cus(s, n_cu));
  if (C < 1) return fail(MOE_EINVAL, "no consumer partition fits this device");
  if (flags == nullptr) {  // the allocation-free variant: flags in the library's scratch array, cleared per call
    if (cfg->mode == 2) return fail(MOE_EINVAL, "mode 2 (return only) needs the flags of an earlier call");
    const int64_t words = ffn_flag_words(s->dtype, s->d, s->f, layout_offsets(s).cap_mtiles);
    if (words > ffn_noalloc_scratch_words())
      return fail(MOE_EINVAL, "this shape's flag buffer needs " + std::to_string(words * 4) +
                                  " bytes, over the allocation-free variant's " +
                                  std::to_string(ffn_noalloc_scratch_words() * 4) + "-byte maximum");
    flags = ffn_noalloc_scratch(dev);
    if (flags == nullptr) return fail(MOE_EHIP, "hipGetSymbolAddress of the scratch array failed");
    if (launch_flags_clear(s->dtype, s->d, s->f, layout_offsets(s).cap_mtiles, flags, (hipStream_t)stream))
      return fail(MOE_EHIP, "flag clear launch failed");
    cfg_v.epoch = 1;  // the flags were just cleared
  }

  FfnLaunch p;
  p.dtype = s->dtype;
  p.R = s->R;
  p.self_rank = s->self_rank;
  p.E = s->num_local_experts;
  p.d = s->d;
  p.f = s->f;
  p.L = L;
  p.x_pad = x_pad;
  p.w_gate_up = w_gate_up;
  p.w_down = w_down;
  p.h = h_ws;
  p.y_pad = y_pad;
  p.recv = recv;
  p.flags = flags;
  p.epoch = cfg->epoch;
  p.band_window = cfg->band_window;
  p.tile_order = cfg->tile_order;
  p.x_tokens = cfg->x_tokens;
  p.gu_out = cfg->gu_out;
  p.join = cfg->mode == 0 && s->dtype == MOE_BF16;
  p.watchdog_ticks = cfg->watchdog_ticks ? cfg->watchdog_ticks : 200000000ull;
  p.timestamps = cfg->timestamps;
  p.cap_mtiles = layout_offsets(s).cap_mtiles;

  if (cfg->mode == 2) {  // return only
    if (launch_ffn_consumer(p, C, st)) return fail(MOE_EHIP, "consumer launch failed");
    return MOE_OK;
  }
  if (cfg->mode == 3) {
    CallEvents ce3;
    const bool timed3 = g_timing && timing_begin(&ce3) == 0;
    if (timed3) ce3.n = 1;
    if (cfg->timestamps && launch_ts_init(cfg->timestamps, 2 + 2 * layout_offsets(s).cap_tiles, st)) {
      if (timed3) ce3.destroy();
      return fail(MOE_EHIP, "launch failed");
    }
    const int rc = ffn_dma(s, L, p, n_cu, dev, st, &ce3, timed3);
    if (timed3) {
      if (rc != MOE_OK) {
        ce3.destroy();
      } else {
        std::lock_guard<std::mutex> lk(g_mu);
        g_events.push_back(ce3);
      }
    }
    return rc;
  }
  CallEvents ce;
  const bool timed = g_timing && timing_begin(&ce) == 0;
  auto failed = [&](const char* m) {
    if (timed) ce.destroy();
    return fail(MOE_EHIP, m);
  };
  hipEvent_t ev0 = nullptr, ev1 = nullptr;  // the next launch's pair
  auto next_pair = [&]() {
    if (timed) {
      ev0 = ce.e[2 * ce.n];
      ev1 = ce.e[2 * ce.n + 1];
      ++ce.n;
    }
  };
  if (cfg->timestamps && launch_ts_init(cfg->timestamps, 2 + 2 * layout_offsets(s).cap_tiles, st))
    return failed("launch failed");
  // overlapped: C consumer workgroups in the producer launch (bf16: the whole FFN; fp32: its second GEMM),
  // producers on the other CUs, each joining the return once its items are done; sequential: producers on
  // every CU, then the return on every CU
  // overlapped bf16 with consumer_cus = 0: the launch picks its own partition (ffn_adaptive_consumers)
  // bf16 with consumer_cus = -1: no partition, the return runs at the launch's tail
  const int n_cons = cfg->mode != 0 ? 0
                     : p.dtype != MOE_BF16 ? C
                     : cfg->consumer_cus == 0 ? -1
                     : cfg->consumer_cus < 0 ? 0 : C;
  next_pair();
  if (launch_ffn_producer(p, n_cu, p.dtype == MOE_BF16 ? n_cons : 0, st, ev0, ev1))
    return failed("producer launch failed");
  if (p.dtype != MOE_BF16) {
    ce.second = timed;
    next_pair();
    if (launch_ffn_producer2(p, n_cu, n_cons, st, ev0, ev1)) return failed("producer launch failed");
  }
  if (cfg->mode == 1) {
    ce.cons = timed;
    next_pair();
    if (launch_ffn_consumer(p, n_cu, st, ev0, ev1)) return failed("consumer launch failed");
  }
  if (timed) {
    std::lock_guard<std::mutex> lk(g_mu);
    g_events.push_back(ce);
  }
  return MOE_OK;
}
}  // namespace

extern "C" {

int moe_expert_ffn_overlap(const moe_shape* s, const moe_layout* L, const void* x_pad, const void* w_gate_up,
                           const void* w_down, void* h_ws, void* y_pad, void* const* recv, uint32_t* flags,
                           const moe_overlap_cfg* cfg, void* stream) {
  if (!flags) return fail(MOE_EINVAL, "null pointer");
  return ffn_overlap(s, L, x_pad, w_gate_up, w_down, h_ws, y_pad, recv, flags, cfg, stream);
}

int moe_expert_ffn_overlap_noalloc(const moe_shape* s, const moe_layout* L, const void* x_pad, const void* w_gate_up,
                                   const void* w_down, void* h_ws, void* y_pad, void* const* recv,
                                   const moe_overlap_cfg* cfg, void* stream) {
  return ffn_overlap(s, L, x_pad, w_gate_up, w_down, h_ws, y_pad, recv, nullptr, cfg, stream);
}

int moe_ffn_schedule(const moe_shape* s, int32_t n_cu, const moe_overlap_cfg* cfg, int32_t n_mtiles,
                     int32_t n_remote_mtiles, const int32_t* mt_hdr, const int32_t* mt_order, int32_t* items,
                     int64_t cap, int64_t* n_items) {
  const std::string e = check_shape(s);
  if (!e.empty()) return fail(MOE_EINVAL, e);
  if (s->dtype != MOE_BF16) return fail(MOE_EINVAL, "the fp32 path runs two plain launches, not an item list");
  if (!cfg || !n_items || n_cu < 2 || n_mtiles < 0 || n_remote_mtiles < 0 || n_remote_mtiles > n_mtiles)
    return fail(MOE_EINVAL, "bad arguments");
  if (n_mtiles > 0 && (!mt_hdr || !mt_order)) return fail(MOE_EINVAL, "null pointer");
  if (cfg->mode != 0 && cfg->mode != 1) return fail(MOE_EINVAL, "mode must be 0 or 1");
  if (cfg->consumer_cus < -1 || cfg->consumer_cus > n_cu / 2 || cfg->band_window < 0 ||
      (cfg->tile_order != 0 && cfg->tile_order != 1))
    return fail(MOE_EINVAL, "consumer_cus, band_window or tile_order out of range");
  std::vector<int32_t> ident;
  const int32_t* mt_order_in = mt_order;
  const int n_remote_in = n_remote_mtiles;
  if (cfg->tile_order == 1) {  // row-tile numbering: no boundary
    ident.resize(n_mtiles);
    for (int i = 0; i < n_mtiles; ++i) ident[i] = i;
    mt_order = ident.data();
    n_remote_mtiles = n_mtiles;
  }
  for (int i = 0; i < n_mtiles; ++i) {
    const int32_t* h = mt_hdr + 4 * (int64_t)i;
    if (h[2] < 0 || h[3] < 1 || h[2] + h[3] > n_mtiles || i < h[2] || i >= h[2] + h[3] || mt_order[i] < 0 ||
        mt_order[i] >= n_mtiles)
      return fail(MOE_EINVAL, "row-tile headers or order out of range");
  }
  // consumer_cus 0: the launch's own rule with default rates, taking every row of the row tiles that hold another
  // owner's row as returned
  int C = cfg->mode != 0 || cfg->consumer_cus < 0 ? 0 : cfg->consumer_cus;
  if (cfg->mode == 0 && cfg->consumer_cus == 0) {
    int64_t m_real = 0, m_ret = 0;
    for (int i = 0; i < n_mtiles; ++i) m_real += mt_hdr[4 * (int64_t)i + 1];
    for (int p = 0; p < n_remote_in; ++p) {
      if (mt_order_in[p] < 0 || mt_order_in[p] >= n_mtiles) return fail(MOE_EINVAL, "row-tile order out of range");
      m_ret += mt_hdr[4 * (int64_t)mt_order_in[p] + 1];
    }
    int n1 = 0, n2 = 0, S = 0;
    ffn_list_dims(s->d, s->f, &n1, &n2, &S);
    C = ffn_adaptive_consumers(n_cu, m_real, m_ret, s->d, s->f, (int64_t)n_mtiles * n1, 0.f, 0.f);
  }
  if (ffn_schedule_host(s->d, s->f, s->num_local_experts, C, n_cu - C, cfg->band_window, n_mtiles, n_remote_mtiles,
                        mt_hdr, mt_order, items, cap, n_items))
    return items == nullptr && cap == 0 ? MOE_OK : fail(MOE_EINVAL, "cap is below the list length");
  return MOE_OK;
}

int moe_combine(const moe_shape* s, const moe_layout* L, const float* topk_w, void* const* recv, void* out,
                void* stream) {
  const std::string e = check_shape(s);
  if (!e.empty()) return fail(MOE_EINVAL, e);
  if (!layout_ok(L)) return fail(MOE_EINVAL, "layout not bound");
  const int64_t T = (int64_t)s->R * s->tokens_per_owner;
  if (T > 0 && (!topk_w || !recv || !out)) return fail(MOE_EINVAL, "null pointer");
  for (int r = 0; T > 0 && r < s->R; ++r)
    if (!recv[r]) return fail(MOE_EINVAL, "null receive buffer");
  CombineLaunch p;
  p.dtype = s->dtype;
  p.R = s->R;
  p.T_o = s->tokens_per_owner;
  p.k = s->top_k;
  p.d = s->d;
  p.E = s->num_local_experts;
  p.G = s->num_global_experts;
  p.L = L;
  p.topk_w = topk_w;
  p.recv = recv;
  p.out = out;
  if (launch_combine(p, (hipStream_t)stream)) return fail(MOE_EHIP, "combine launch failed");
  return MOE_OK;
}

int64_t moe_bwd_flags_count(const moe_shape* s) {
  if (!check_shape(s).empty() || s->dtype != MOE_BF16 || s->f % 128) return -1;
  return bwd_flag_words(s->d, s->f, layout_offsets(s).cap_mtiles);
}

int moe_expert_ffn_backward(const moe_shape* s, const moe_layout* L, const moe_bwd_args* b, uint32_t* flags,
                            const moe_overlap_cfg* cfg, void* stream) {
  const std::string e = check_shape(s);
  if (!e.empty()) return fail(MOE_EINVAL, e);
  if (s->dtype != MOE_BF16) return fail(MOE_EINVAL, "the backward pass is for bf16");
  if (s->f % 128) return fail(MOE_EINVAL, "the backward pass needs f to be a multiple of 128");
  if (!layout_ok(L) || !b || !cfg || !flags) return fail(MOE_EINVAL, "null layout, arguments, flags or cfg");
  if (L->cap_tiles * s->tile_m != L->cap_rows) return fail(MOE_EINVAL, "layout bound for another tile_m");
  if ((L->cap_rows + 256) * 4ll * s->f >= (1ll << 32)) return fail(MOE_EINVAL, "rows x 2f too large for 32-bit offsets");
  const int64_t T = (int64_t)s->R * s->tokens_per_owner;
  if (!b->x_pad || !b->w_gate_up || !b->w_down || !b->dy_pad || !b->dh_ws || !b->h_ws || !b->dgu_ws || !b->dx_pad ||
      !b->dx_recv || !b->dw_gate_up || !b->dw_down || (T > 0 && (!b->topk_idx || !b->topk_w || !b->d_out)))
    return fail(MOE_EINVAL, "null pointer");
  for (int r = 0; r < s->R; ++r)
    if (!b->dx_recv[r]) return fail(MOE_EINVAL, "null receive buffer");
  if ((uintptr_t)flags % 8 != 0) return fail(MOE_EINVAL, "flags must be 8-byte aligned");
  if (cfg->epoch == 0) return fail(MOE_EINVAL, "epoch must be nonzero");
  if (cfg->mode != 0 && cfg->mode != 1) return fail(MOE_EINVAL, "the backward pass runs in mode 0 or 1");
  if (cfg->x_tokens || cfg->gu_out) return fail(MOE_EINVAL, "x_tokens and gu_out are for the forward call");
  hipStream_t st = (hipStream_t)stream;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(MOE_EHIP, "hipGetDevice failed");
  const int n_cu = device_cus(dev);
  if (n_cu <= 0) return fail(MOE_EHIP, "cannot query the CU count");
  if (cfg->consumer_cus < -1 || cfg->consumer_cus > n_cu / 2)
    return fail(MOE_EINVAL, "consumer_cus must be -1 (none), 0 (library default) or in [1, CUs/2]");
  // the default: no consumer workgroups (every workgroup takes the copy units once the weight-gradient tiles are
  // handed out).  On one device the dX return is an HBM copy of about 2% of the launch's time on the whole chip, and
  // C workgroups returning rows during the weight-gradient tiles slowed the launch more than that (DeepSeek-V3-like
  // shard: 7.17 ms with 8 against 6.97 + 0.17 ms for the producers alone and then the return)
  const int C = cfg->consumer_cus > 0 ? cfg->consumer_cus : 0;
  BwdLaunch p;
  p.R = s->R;
  p.E = s->num_local_experts;
  p.d = s->d;
  p.f = s->f;
  p.k = s->top_k;
  p.M = s->tile_m;
  p.lo = s->self_rank * s->num_local_experts;
  p.self_rank = s->self_rank;
  p.L = L;
  p.x_pad = b->x_pad;
  p.w_gate_up = b->w_gate_up;
  p.w_down = b->w_down;
  p.topk_idx = b->topk_idx;
  p.topk_w = b->topk_w;
  p.d_out = b->d_out;
  p.dy_pad = b->dy_pad;
  p.dh_ws = b->dh_ws;
  p.h_ws = b->h_ws;
  p.dgu_ws = b->dgu_ws;
  p.gu = b->gu;
  p.dx_pad = b->dx_pad;
  p.dx_recv = b->dx_recv;
  p.dw_gate_up = b->dw_gate_up;
  p.dw_down = b->dw_down;
  p.flags = flags;
  p.epoch = cfg->epoch;
  p.watchdog_ticks = cfg->watchdog_ticks ? cfg->watchdog_ticks : 200000000ull;
  p.cap_mtiles = layout_offsets(s).cap_mtiles;
  if (launch_bwd_dy(p, st)) return fail(MOE_EHIP, "dY launch failed");
  CallEvents ce;
  const bool timed = g_timing && timing_begin(&ce) == 0;
  hipEvent_t ev0 = timed ? ce.e[0] : nullptr, ev1 = timed ? ce.e[1] : nullptr;
  if (timed) ce.n = 1;
  const int n_cons = cfg->mode == 0 ? C : 0;
  if (launch_bwd_ffn(p, n_cu, n_cons, cfg->mode == 0, st, ev0, ev1)) {
    if (timed) ce.destroy();
    return fail(MOE_EHIP, "backward launch failed");
  }
  if (cfg->mode == 1) {
    if (timed) {
      ce.n = 2;
      ce.cons = true;
    }
    if (launch_bwd_consumer(p, n_cu, st, timed ? ce.e[2] : nullptr, timed ? ce.e[3] : nullptr)) {
      if (timed) ce.destroy();
      return fail(MOE_EHIP, "consumer launch failed");
    }
  }
  if (timed) {
    std::lock_guard<std::mutex> lk(g_mu);
    g_events.push_back(ce);
  }
  return MOE_OK;
}

int moe_combine_backward(const moe_shape* s, const moe_layout* L, const void* d_out, void* const* y_recv,
                         void* const* dx_recv, void* dx, float* dw_route, void* stream) {
  const std::string e = check_shape(s);
  if (!e.empty()) return fail(MOE_EINVAL, e);
  if (s->dtype != MOE_BF16) return fail(MOE_EINVAL, "the backward pass is for bf16");
  if (!layout_ok(L)) return fail(MOE_EINVAL, "layout not bound");
  const int64_t T = (int64_t)s->R * s->tokens_per_owner;
  if (T > 0 && (!d_out || !y_recv || !dx_recv || !dx || !dw_route)) return fail(MOE_EINVAL, "null pointer");
  for (int r = 0; T > 0 && r < s->R; ++r)
    if (!y_recv[r] || !dx_recv[r]) return fail(MOE_EINVAL, "null receive buffer");
  BwdLaunch p{};
  p.R = s->R;
  p.E = s->num_local_experts;
  p.d = s->d;
  p.k = s->top_k;
  p.L = L;
  p.d_out = d_out;
  p.dx_recv = dx_recv;
  if (launch_bwd_combine(p, s->tokens_per_owner, s->num_global_experts, L->combine_plan, y_recv, dx, dw_route,
                         (hipStream_t)stream))
    return fail(MOE_EHIP, "combine backward launch failed");
  return MOE_OK;
}

}  // extern "C"
