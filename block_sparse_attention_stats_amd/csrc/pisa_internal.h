// Host-side interface between the C ABI (pisa_abi.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pisa {

// Byte offsets of the regions of the caller's workspace (all 256-aligned).
struct WsLayout {
  size_t kp, vp;      // K-format / V-format sub-tiles of K and V: [BH][n][blk/64][64*D]
  size_t kbp, vbp;    // K-format k̄ / V-format ΣV tiles: [BH][ceil(n/64)][64*D]
  size_t hbt;         // H̄ᵀ operand chunks: [BH][D*D]
  size_t hpart;       // fp32 partial Σ_j H_j per chunk of blocks: [BH][nch][D][D]
  size_t scores;      // fp64 routing scores of a chunk of heads: [heads][n][n]; empty when
                      // n <= kRouteMaxBlocks (k_route keeps them on chip)
  size_t kmax2;       // fp32 largest squared key norm per run of blocks: [BH][nch]
  size_t redo;        // int32 count + list of query tiles the careful kernel recomputes
  size_t sync;        // int32 arrival counters of the fast kernel's generation barrier, one per XCD
  size_t total;       // bytes needed by stats + select + forward
  size_t dense_total; // bytes needed by the dense baseline (kp + vp)
  int n, spb, nct, cb, nch, esz;
  long bh;
};

struct StatsArgs {
  const uint8_t *q, *k, *v;
  double *qbar, *kbar, *vsum, *mnorm;
  double* hbar;
  uint8_t *kp, *vp, *kbp, *vbp, *hbt;
  float* hpart;
  float* kmax2;
  // Token `row` of head bh: rows below L0 are in q, k, v at byte offset
  // (bh / H) * stride_b + (bh % H) * stride_h + row * stride_l; rows from L0
  // on are in q1, k1, v1, at the same form of offset with stride1_* and
  // row - L0 (the second segment of a joint sequence; L0 = L when there is none)
  size_t stride_b, stride_h, stride_l;
  const uint8_t *q1, *k1, *v1;
  size_t stride1_b, stride1_h, stride1_l;
  int H, L0;
  int L, n, blk, cb, nch, nct;
};

struct ScoreArgs {
  const double *qbar, *kbar, *mnorm;
  double* scores;
  double scale, cov_weight;
  int n, sink_block;  // sink_block < 0: none
};

struct TopkArgs {
  const double* scores;
  int32_t* idx;
  int n, topk;
};

// Scores and top-k in one pass (rows of at most kRouteMaxBlocks blocks).
struct RouteArgs {
  const double *qbar, *kbar, *mnorm;
  int32_t* idx;
  double scale, cov_weight;
  int n, topk, sink_block;  // sink_block < 0: none
  int nrt;                  // workgroups per head: 16 query blocks each
  long total;               // workgroups in all
};

struct FwdArgs {
  const uint8_t* q;
  uint8_t* o;
  const uint8_t *kp, *vp, *kbp, *vbp, *hbt;
  const int32_t* idx;  // nullptr: every key block (dense)
  const float* kmax2;  // [BH][nch] largest squared key norm per run of blocks
  int* redo;           // [0]: count, [1..]: query tiles left to the careful kernel
  int* sync;           // arrival counters of the fast kernel's generation barrier (kSyncCounters)
  long nwg;            // workgroups per generation of the fast kernel (as many as are resident)
  int sync_ticks;      // longest wait at a generation barrier, in 100 MHz ticks
  long total;
  int L, n, blk, topk, n_last, nct, nch;
  float cs;     // scale * log2(e)
  float scale;
  int first_order, tail;
  int per_block;  // per-block first-order variant (first_order is then 0)
  size_t stride_b, stride_h, stride_l;  // q and o addressing, as in StatsArgs
  const uint8_t* q1;                    // second segment of q and o
  uint8_t* o1;
  size_t stride1_b, stride1_h, stride1_l;
  int H, L0;
  float* lse;  // [BH][L]: natural log of each row's denominator D_t, or nullptr
};

// Backward pass of the zeroth-order variant.
struct BwdArgs {
  const uint8_t *q, *k, *v, *o, *dout;  // [B,H,L,D] or [B,L,H,D], I/O dtype
  uint8_t *dq, *dk, *dv;
  size_t stride_b, stride_h, stride_l;  // byte strides, as in StatsArgs
  int H;
  const double *kbar, *vsum;  // block statistics of the forward pass: [BH][n][D] fp64
  const int32_t* idx;         // [BH][n][topk]
  uint32_t* selmap;           // [BH][n][W]: bit j of row i set when query block i selects j
  float *lse, *delta;         // [BH][n*blk]: log2 of each row's denominator, dO·o
  const float* lse_in;        // [BH][L]: ln D_t from the forward pass, or nullptr
  float *dkbar, *dvsum;       // [BH][n][D]: gradients of k̄_j and ΣV_j
  uint8_t *kbt, *vbt;         // [BH][nct*64][D]: k̄_j and ΣV_j in the I/O dtype, zero past n
  float *dkbar_p, *dvsum_p;   // [cparts][BH][nct*64][D]: partial centroid gradients (cparts > 1)
  int cparts;                 // query-block ranges the centroid gradients are split into
  int L, n, blk, n_last, nct, topk, W;
  float scale;
  int* sync;                  // k_bwd_dq's count of workgroups past their selected sub-tiles
  int sync_ticks;             // longest wait at k_bwd_dq's generation barrier, 100 MHz ticks
  long total;                 // query tiles (= key sub-tiles): bh * n * (blk / 64)
  long nwg_dq, nwg_dkv;       // resident workgroups of k_bwd_dq / k_bwd_dkv (a generation)
};

// Byte offsets of the backward workspace regions (all 256-aligned).
struct BwdLayout {
  size_t selmap, lse, delta, dkbar, dvsum, kbt, vbt, dkbar_p, dvsum_p, sync, total;
  int cparts;
};

enum StatsMode { kStatsFull = 0, kStatsMnorm = 1, kStatsPackOnly = 2 };

// Each returns hipGetLastError() after enqueueing.
hipError_t launch_block_stats(int dtype, int D, int mode, const StatsArgs& a, long bh,
                              hipStream_t s);
hipError_t launch_hbar_reduce(int dtype, int D, const StatsArgs& a, long bh, hipStream_t s);
// M_j = ||H_j − H̄||_2 per block (after the statistics and H̄ are complete).
hipError_t launch_mnorm_spectral(int dtype, int D, const StatsArgs& a, long bh, hipStream_t s);
hipError_t launch_scores(int D, const ScoreArgs& a, long bh, hipStream_t s);
hipError_t launch_topk(const TopkArgs& a, long rows, hipStream_t s);
hipError_t launch_route(int D, const RouteArgs& a, hipStream_t s);
constexpr int kRouteMaxBlocks = 1280;  // longest row k_route keeps in LDS (80 KB per workgroup)
// Fast pass, then the careful pass over the query tiles the fast pass queued.
hipError_t launch_fwd(int dtype, int D, const FwdArgs& a, hipStream_t s);
// The bf16 fused pass and dense baseline (not the per-block first-order
// variant), from the unit of k_fwd.hip built with MFMA results in VGPRs.
hipError_t launch_fwd_bf16(int D, const FwdArgs& a, hipStream_t s);

// Backward of the zeroth-order variant: selection bitmap, dq (with the row
// statistics), centroid gradients, then dk and dv.
hipError_t launch_bwd(int dtype, int D, const BwdArgs& a, long bh, hipStream_t s);

constexpr int kSyncCounters = 8;  // one generation-barrier counter per XCD
constexpr int kMaxBlocks = 8192;  // routing keeps one score row per workgroup in LDS

}  // namespace pisa
