// Internal launch interface between the C-ABI host code and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_overlap.h"

struct LayoutLaunch {
  const int32_t* topk_idx;
  const void* x;
  void* x_pad;
  moe_layout* L;
  int R, T_o, G, k, lo, E, M, mgb, self_rank, mt_rows;
  int64_t row_bytes;
};

// Expert FFN launch description (producer GEMMs and the consumer role of the second GEMM's launch).
struct FfnLaunch {
  int dtype;  // moe_dtype
  int R, E, d, f;
  int self_rank;  // owner whose rows the producer stores into its receive buffer itself
  const moe_layout* L;
  const void* x_pad;
  const void* w_gate_up;
  const void* w_down;
  void* h;
  void* y_pad;
  void* const* recv;
  uint32_t* flags;
  uint32_t epoch;
  int band_window;
  int tile_order;  // 0: remote first (the layout's mt_order), 1: row-tile numbering
  int join = 0;  // bf16: the producer launch runs the return too (overlapped mode)
  const void* x_tokens = nullptr;  // bf16: token rows; non-null: the launch lands x_pad's rows itself
  float* gu_out = nullptr;         // bf16: non-null: the first GEMM's items also store g | u (fp32) of their rows
  int item_begin = 0, item_end = -1;  // bf16: run list indices [item_begin, item_end) only (GEMM1 first, no
                                      // half-width round); item_end < 0: the whole list
  uint64_t watchdog_ticks;
  uint64_t* timestamps;
  int64_t cap_mtiles;
};

struct CombineLaunch {
  int dtype;
  int R, T_o, k, d;
  int E, G;  // local and global experts (the expected share of local slots)
  const moe_layout* L;
  const float* topk_w;
  void* const* recv;
  void* out;
};

int launch_route(int T, int G, int k, const float* logits, int32_t* topk_idx, float* topk_w, hipStream_t st);
int launch_layout(const LayoutLaunch& p, hipStream_t st);

// GEMM row-tile height (rows) of the producer: the layout packs up to this many real rows into a row tile.
int ffn_gemm_bm(int dtype);
// Output tile width of the second GEMM (y): flags are one per (row tile, column tile).
int ffn_gemm2_bn(int dtype, int d);
// k-splits of a second-GEMM tile (bf16; 1 for fp32).
int ffn_splits(int dtype, int d, int f);
// 4-byte words of the FFN flag buffer: y-tile flags first, then (bf16) h-tile flags, split flags and the
// fp32 partial sums of the k-splits.
int64_t ffn_flag_words(int dtype, int d, int f, int64_t cap_mtiles);
// Producer launch, one workgroup per CU, whose first `n_cons` workgroups run the consumer role.  bf16: the
// whole FFN in one launch (launch_ffn_producer2 is a no-op); fp32: the first GEMM, then the second GEMM with the
// consumer workgroups.  Non-null ev0 / ev1 take the launch's own start and end times (hipExtLaunchKernel), with
// no marker in the stream.
int launch_ffn_producer(const FfnLaunch& p, int grid, int n_cons, hipStream_t st, hipEvent_t ev0 = nullptr,
                        hipEvent_t ev1 = nullptr);
int launch_ffn_producer2(const FfnLaunch& p, int grid, int n_cons, hipStream_t st, hipEvent_t ev0 = nullptr,
                         hipEvent_t ev1 = nullptr);
// The consumer alone (`n_cons` workgroups).
int launch_ffn_consumer(const FfnLaunch& p, int n_cons, hipStream_t st, hipEvent_t ev0 = nullptr,
                        hipEvent_t ev1 = nullptr);
// The fused bf16 launch's item list on the host (item_list.h), as moe_ffn_schedule reports it: for list index i,
// items[8 i ..] = {workgroup, its sequence number there, kind, row tile, column tile, split, half, target}.  -1 if
// cap < the list length (*n_out holds it either way).
int ffn_schedule_host(int d, int f, int E, int n_cons, int n_producers, int band_window, int n_mt, int n_rem,
                      const int32_t* mt_hdr, const int32_t* mt_order, int32_t* items, int64_t cap, int64_t* n_out);
// n_rem and mt_order of a launch: the layout's (remote first), or every tile in number order (tile_order = 1)
// Column tiles of the two GEMMs and k-splits of the bf16 launch for hidden d and FFN width f.
void ffn_list_dims(int d, int f, int* n_nt1, int* n_nt2, int* S);
// The allocation-free variant's flag buffer: its size in 4-byte words, and its device address on device `dev` (the
// current device; looked up once per device), null if the lookup fails.
int64_t ffn_noalloc_scratch_words();
uint32_t* ffn_noalloc_scratch(int dev);
// Zeroes the words of a flag buffer that a call reads before writing (flags, counters), on stream st.
int launch_flags_clear(int dtype, int d, int f, int64_t cap_mtiles, uint32_t* flags, hipStream_t st);
// Resets the n timestamp entries of a call (starts to the largest value, ends to zero).
int launch_ts_init(uint64_t* timestamps, int64_t n, hipStream_t st);
int launch_combine(const CombineLaunch& p, hipStream_t st);

// Backward pass of the expert FFN (bwd.hip).
struct BwdLaunch {
  int R, E, d, f, k, M, lo, self_rank;
  const moe_layout* L;
  const void* x_pad;
  const void* w_gate_up;
  const void* w_down;
  const int32_t* topk_idx;
  const float* topk_w;
  const void* d_out;
  void* dy_pad;
  float* dh_ws;
  void* h_ws;
  void* dgu_ws;
  const float* gu = nullptr;  // g | u stored by the forward (null: recomputed)
  void* dx_pad;
  void* const* dx_recv;
  float* dw_gate_up;
  float* dw_down;
  uint32_t* flags;
  uint32_t epoch;
  uint64_t watchdog_ticks;
  int64_t cap_mtiles;
};
// 4-byte words of the backward flag buffer.
int64_t bwd_flag_words(int d, int f, int64_t cap_mtiles);
// dY rows of the padded layout (bf16 of w dOut).
int launch_bwd_dy(const BwdLaunch& p, hipStream_t st);
// The backward launch on `grid` CUs: the first n_cons workgroups run the dX return only; with join, the others take
// copy units once their items are done.
int launch_bwd_ffn(const BwdLaunch& p, int grid, int n_cons, int join, hipStream_t st, hipEvent_t ev0 = nullptr,
                   hipEvent_t ev1 = nullptr);
// The dX return alone (`n_cons` workgroups).
int launch_bwd_consumer(const BwdLaunch& p, int n_cons, hipStream_t st, hipEvent_t ev0 = nullptr,
                        hipEvent_t ev1 = nullptr);
// The combine's backward: dx (bf16 [T, d]) and the routing weights' gradient dw (fp32 [T, k]); G global experts (with
// p.E, the expected share of local slots, which sets the loads' cache policy).
int launch_bwd_combine(const BwdLaunch& p, int T_o, int G, const int32_t* plan, void* const* y_recv, void* dx,
                       float* dw, hipStream_t st);
// A nonzero value distinct for every launch that opens a copy-unit counter.
uint32_t next_stamp();
