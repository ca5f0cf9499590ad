// Per-query-block top-k routing (gist.science technical summary of arXiv
// 2602.01077, section 2 "Covariance-Aware Routing"; the authors' README,
// "Attention sink for MMDiT").
//
// Scores: S_ij = scale * q̄_i·k̄_j + cov_weight * M_j in fp64 over (query block,
//   key block) tiles (n x n x D per head: small next to the fused pass); the
//   sink column gets +infinity. Both paths form them with the same products
//   on the fp64 matrix cores.
// Rows of up to kRouteMaxBlocks blocks take k_route, which keeps the scores on
// chip (see there); longer rows take k_scores_mfma, whose scores pass through
// the workspace, and then k_topk_wave or k_topk.
// Top-k of a row: the k-th largest key T is narrowed down by an MSB-first
//   radix select over order-preserving 64-bit keys, stopping early once the
//   bucket that holds it is to be taken whole; then every key above T and the
//   lowest-index keys equal to it are taken, and the indices emitted ascending.
//   k_topk_wave (rows of 1281 to 2048 blocks): one wavefront per row, its keys in
//   registers; each pass's 8-bit digit starts at the highest bit in which the
//   remaining candidates still differ, so no pass is spent on the sign and
//   exponent bits they share. k_topk (longer rows): one workgroup per row, the
//   keys in LDS, fixed 8-bit digits. Both return the same set.
#include "pisa_dev.h"
#include "pisa_internal.h"

namespace pisa {

typedef double f64x4 __attribute__((ext_vector_type(4)));

// k_scores_mfma: the pooled scores on the fp64 matrix cores, for rows longer than
// kRouteMaxBlocks.
// Each wavefront computes 16·TR x 16·TC (query block, key block) pairs as
// TR x TC products of v_mfma_f64_16x16x4f64 (A: row m = lane % 16,
// k = lane / 16; B: k = lane / 16, column = lane % 16; D: element r of a
// lane is row lane / 16 + 4r, column lane % 16); four wavefronts in a 2 x 2
// square make a workgroup. The k index is mapped so that each lane reads four
// consecutive d of its q̄ / k̄ row with one 32-byte load: in step s of a
// 16-wide chunk at d0, k = g stands for d = d0 + 4g + s. Operands come
// straight from global memory (the L2 holds a head's q̄ and k̄); the next chunk
// is loaded while the current one is multiplied.
template <int D, int TR, int TC>
__global__ __launch_bounds__(256) void k_scores_mfma(ScoreArgs a) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int r0 = blockIdx.y * 32 * TR + 16 * TR * (wv >> 1);
  const int c0 = blockIdx.x * 32 * TC + 16 * TC * (wv & 1);
  if (r0 >= a.n || c0 >= a.n) return;
  const long bh = blockIdx.z;
  const double* qb = a.qbar + (size_t)bh * a.n * D + 4 * g;
  const double* kb = a.kbar + (size_t)bh * a.n * D + 4 * g;
  const double* pa[TR];
  const double* pb[TC];
#pragma unroll
  for (int t = 0; t < TR; ++t)  // rows and columns past n: computed, not stored
    pa[t] = qb + (size_t)min(r0 + 16 * t + c, a.n - 1) * D;
#pragma unroll
  for (int u = 0; u < TC; ++u) pb[u] = kb + (size_t)min(c0 + 16 * u + c, a.n - 1) * D;
  f64x4 acc[TR][TC];
#pragma unroll
  for (int t = 0; t < TR; ++t)
#pragma unroll
    for (int u = 0; u < TC; ++u) acc[t][u] = f64x4{0.0, 0.0, 0.0, 0.0};
  f64x4 A[TR], B[TC];
#pragma unroll
  for (int t = 0; t < TR; ++t) A[t] = *reinterpret_cast<const f64x4*>(pa[t]);
#pragma unroll
  for (int u = 0; u < TC; ++u) B[u] = *reinterpret_cast<const f64x4*>(pb[u]);
#pragma unroll
  for (int d0 = 0; d0 < D; d0 += 16) {
    f64x4 An[TR], Bn[TC];
    if (d0 + 16 < D) {
#pragma unroll
      for (int t = 0; t < TR; ++t) An[t] = *reinterpret_cast<const f64x4*>(pa[t] + d0 + 16);
#pragma unroll
      for (int u = 0; u < TC; ++u) Bn[u] = *reinterpret_cast<const f64x4*>(pb[u] + d0 + 16);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int t = 0; t < TR; ++t)
#pragma unroll
        for (int u = 0; u < TC; ++u)
          acc[t][u] = __builtin_amdgcn_mfma_f64_16x16x4f64(A[t][s], B[u][s], acc[t][u], 0, 0, 0);
    if (d0 + 16 < D) {
#pragma unroll
      for (int t = 0; t < TR; ++t) A[t] = An[t];
#pragma unroll
      for (int u = 0; u < TC; ++u) B[u] = Bn[u];
    }
  }
  double* out = a.scores + (size_t)bh * a.n * a.n;
#pragma unroll
  for (int u = 0; u < TC; ++u) {
    const int j = c0 + 16 * u + c;
    if (j >= a.n) continue;
    const double cov = a.cov_weight != 0.0 ? a.cov_weight * a.mnorm[bh * a.n + j] : 0.0;
#pragma unroll
    for (int t = 0; t < TR; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = r0 + 16 * t + g + 4 * r;
        if (i >= a.n) continue;
        double sc = a.scale * acc[t][u][r];
        if (a.cov_weight != 0.0) sc = sc + cov;
        if (j == a.sink_block) sc = __builtin_huge_val();
        out[(size_t)i * a.n + j] = sc;
      }
  }
}

// Monotone map from fp64 to uint64: larger value -> larger key (-0 == +0).
__device__ inline unsigned long long order_key(double x) {
  if (x == 0.0) x = 0.0;
  const unsigned long long u = __double_as_longlong(x);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// Inclusive prefix sum over the 256 threads of the block.
__device__ inline int block_scan_incl(int v, int* wsum) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(v, o);
    if (lane >= o) v += y;
  }
  __syncthreads();
  if (lane == 63) wsum[wv] = v;
  __syncthreads();
  for (int w = 0; w < wv; ++w) v += wsum[w];
  return v;
}

__global__ __launch_bounds__(256) void k_topk(TopkArgs a) {
  extern __shared__ unsigned long long keys[];
  __shared__ int hist[256];
  __shared__ int wsum[4];
  __shared__ int pick_digit, pick_gt, pick_cnt;
  const int tid = threadIdx.x;
  const long row = blockIdx.x;
  const int n = a.n, k = a.topk;
  int32_t* out = a.idx + row * (long)k;
  if (k >= n) {
    for (int j = tid; j < n; j += 256) out[j] = j;
    return;
  }
  const double* S = a.scores + row * (long)n;
  for (int j = tid; j < n; j += 256) keys[j] = order_key(S[j]);
  unsigned long long prefix = 0, pmask = 0;
  int kk = k;
  for (int shift = 56; shift >= 0; shift -= 8) {
    hist[tid] = 0;
    __syncthreads();
    for (int j = tid; j < n; j += 256) {
      const unsigned long long key = keys[j];
      if ((key & pmask) == prefix) atomicAdd(&hist[(int)((key >> shift) & 255)], 1);
    }
    __syncthreads();
    // thread t looks at digit 255 - t: incl = count of candidates with digit >= it
    const int dg = 255 - tid;
    const int c = hist[dg];
    const int incl = block_scan_incl(c, wsum);
    const int gt = incl - c;
    if (gt < kk && kk <= incl) {
      pick_digit = dg;
      pick_gt = gt;
      pick_cnt = c;
    }
    __syncthreads();
    prefix |= (unsigned long long)pick_digit << shift;
    pmask |= 255ull << shift;
    kk -= pick_gt;
    const bool whole_bucket = (pick_cnt == kk);
    __syncthreads();
    // every key left in the k-th key's bucket is selected: the remaining bits
    // cannot change the set (and there is no tie to break)
    if (whole_bucket) break;
  }
  // Keys whose digits so far exceed the prefix are selected, and of those equal
  // to it the kk lowest-index ones (after all 8 passes: all keys > T, the k-th
  // largest key, and the kk lowest-index keys == T).
  const int per = (n + 255) / 256, lo = min(n, tid * per), hi = min(n, lo + per);
  int ceq = 0;
  for (int j = lo; j < hi; ++j) ceq += ((keys[j] & pmask) == prefix);
  int eq_before = block_scan_incl(ceq, wsum) - ceq;
  int cnt = 0;
  {
    int r = eq_before;
    for (int j = lo; j < hi; ++j) {
      const unsigned long long key = keys[j] & pmask;
      const bool sel = key > prefix || (key == prefix && r++ < kk);
      cnt += sel;
    }
  }
  int pos = block_scan_incl(cnt, wsum) - cnt;
  {
    int r = eq_before;
    for (int j = lo; j < hi; ++j) {
      const unsigned long long key = keys[j] & pmask;
      const bool sel = key > prefix || (key == prefix && r++ < kk);
      if (sel) out[pos++] = j;
    }
  }
}

// Wave-wide OR / AND of a 64-bit value.
__device__ inline unsigned long long wave_or64(unsigned long long x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x |= __shfl_xor(x, o);
  return x;
}
__device__ inline unsigned long long wave_and64(unsigned long long x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x &= __shfl_xor(x, o);
  return x;
}

// Orders the LDS accesses of one wavefront against each other (the DS unit
// runs a wave's operations in issue order; the fence keeps the compiler from
// moving them).
__device__ inline void wave_lds_order() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront"); }

// One wavefront per row; key j lives in lane j % 64, slot j / 64 (KPL slots).
template <int KPL>
__global__ __launch_bounds__(256) void k_topk_wave(TopkArgs a, long rows) {
  __shared__ int4 hist_all[4][64];  // 256 digit counts per wavefront
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const long row = (long)blockIdx.x * 4 + wv;
  if (row >= rows) return;
  int4* hist4 = hist_all[wv];
  int* hist = reinterpret_cast<int*>(hist4);
  const int n = a.n, k = a.topk;
  int32_t* out = a.idx + row * (long)k;
  if (k >= n) {
    for (int j = lane; j < n; j += 64) out[j] = j;
    return;
  }
  const double* S = a.scores + row * (long)n;
  // all loads in flight at once: slots past the end read the row's last score
  double x[KPL];
#pragma unroll
  for (int s = 0; s < KPL; ++s) x[s] = S[min(s * 64 + lane, n - 1)];
  unsigned long long key[KPL];
#pragma unroll
  for (int s = 0; s < KPL; ++s) key[s] = order_key(x[s]);
  unsigned long long prefix = 0, pmask = 0;
  int kk = k;
  for (;;) {
    // bits in which the candidates (keys matching prefix under pmask) differ
    unsigned long long vor = 0, vand = ~0ull;
#pragma unroll
    for (int s = 0; s < KPL; ++s) {
      if (s * 64 + lane < n && (key[s] & pmask) == prefix) {
        vor |= key[s];
        vand &= key[s];
      }
    }
    vor = wave_or64(vor);
    vand = wave_and64(vand);
    const unsigned long long diff = vor ^ vand;
    if (diff == 0) {  // every candidate equals T: ties go by index below
      prefix = vand;
      pmask = ~0ull;
      break;
    }
    const int top = 63 - __clzll(diff);
    const int shift = top >= 7 ? top - 7 : 0;
    pmask = top == 63 ? 0ull : (~0ull << (top + 1));  // shared by every candidate
    prefix = vand & pmask;
    hist4[lane] = make_int4(0, 0, 0, 0);
    wave_lds_order();
#pragma unroll
    for (int s = 0; s < KPL; ++s)
      if (s * 64 + lane < n && (key[s] & pmask) == prefix)
        atomicAdd(&hist[(int)((key[s] >> shift) & 255)], 1);
    wave_lds_order();
    // lane l holds digits 255-4l .. 252-4l, counted from the top
    const int4 h = hist4[63 - lane];
    const int c[4] = {h.w, h.z, h.y, h.x};
    const int tot = c[0] + c[1] + c[2] + c[3];
    int incl = tot;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    const int before = incl - tot;
    const bool mine = before < kk && kk <= incl;
    int dg = 0, gt = 0, cnt = 0;
    if (mine) {
      int g = before;
      bool found = false;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (!found && g + c[u] >= kk) {
          dg = 255 - 4 * lane - u;
          gt = g;
          cnt = c[u];
          found = true;
        }
        g += c[u];
      }
    }
    const int src = __ffsll((unsigned long long)__ballot(mine)) - 1;
    dg = __shfl(dg, src);
    gt = __shfl(gt, src);
    cnt = __shfl(cnt, src);
    prefix |= (unsigned long long)dg << shift;
    pmask |= 255ull << shift;
    kk -= gt;
    wave_lds_order();  // the next pass clears the counts only after they are read
    if (cnt == kk || shift == 0) break;
  }
  // every key above prefix, and the kk lowest-index keys equal to it
  const unsigned long long lt = (1ull << lane) - 1ull;
  int eq_seen = 0, pos = 0;
#pragma unroll
  for (int s = 0; s < KPL; ++s) {
    const int j = s * 64 + lane;
    const unsigned long long km = key[s] & pmask;
    const bool valid = j < n;
    const bool above = valid && km > prefix, eq = valid && km == prefix;
    const unsigned long long beq = __ballot(eq);
    const bool sel = above || (eq && eq_seen + __popcll(beq & lt) < kk);
    const unsigned long long bsel = __ballot(sel);
    const int at = pos + __popcll(bsel & lt);
    if (sel && at < k) out[at] = j;  // exactly k are selected; the bound only guards the row
    pos += __popcll(bsel);
    eq_seen += __popcll(beq);
  }
}

// ---------------------------------------------------------------------------
// k_route: the scores of 16 query blocks and their top-k in one pass, for rows
// of up to kRouteMaxBlocks blocks; the score matrix never leaves the chip.
//
// Phase 1: the workgroup's eight wavefronts share out the key blocks in units
// of 32 and form q̄_i·k̄_j for the 16 rows on the fp64 matrix cores, in the
// same products and order as k_scores_mfma. Of each score's order-preserving
// 64-bit key only the upper 32 bits are kept, in LDS: 16 rows of up to 1280
// keys is 80 KB, so two workgroups share a CU and each SIMD runs four
// wavefronts (the fp64 matrix cores reach about 35 TFLOP/s with one wavefront
// per SIMD and 46-48 with two to four; measured on MI355X).
// Phase 2: one wavefront per row selects on those 32 bits by a binary radix
// select that counts with wave-wide sums (no LDS traffic). Where the k-th place falls
// inside a run of keys whose upper halves are equal and only part of the run
// is taken (a near or exact tie), the wavefront forms the run's scores again,
// bit for bit as before, and selects within the run on the lower 32 bits; keys
// equal in all 64 bits go to the lower index, as everywhere else.

constexpr int kRouteRows = 16;

// The raw products of TU tiles of 16 key blocks from col0: acc[u][r] is
// q̄_i·k̄_j for row i = i0 + g + 4r and key block j = col0 + 16u + c
// (lane = 16g + c), as 16 x 16 products of v_mfma_f64_16x16x4f64 over d in
// chunks of 16 (k = g stands for d = d0 + 4g + t in step t). A holds the 16
// rows' q̄ in that form; columns past the end repeat the last key block
// (formed, never stored). Each product is the same chain of MFMAs whatever TU
// and col0, so a product formed again has the same bits.
template <int D, int TU = 4>
__device__ __forceinline__ void route_dots(const f64x4 (&A)[D / 16], const double* kb, int col0, int n,
                                           int g, int c, f64x4 (&acc)[TU]) {
  const double* pb[TU];
  f64x4 B[TU];
#pragma unroll
  for (int u = 0; u < TU; ++u) {
    pb[u] = kb + (size_t)min(col0 + 16 * u + c, n - 1) * D + 4 * g;
    acc[u] = f64x4{0.0, 0.0, 0.0, 0.0};
    B[u] = *reinterpret_cast<const f64x4*>(pb[u]);
  }
#pragma unroll
  for (int ch = 0; ch < D / 16; ++ch) {
    f64x4 Bn[TU];
    if (ch + 1 < D / 16) {
#pragma unroll
      for (int u = 0; u < TU; ++u) Bn[u] = *reinterpret_cast<const f64x4*>(pb[u] + 16 * (ch + 1));
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int u = 0; u < TU; ++u)
        acc[u] = __builtin_amdgcn_mfma_f64_16x16x4f64(A[ch][t], B[u][t], acc[u], 0, 0, 0);
    if (ch + 1 < D / 16) {
#pragma unroll
      for (int u = 0; u < TU; ++u) B[u] = Bn[u];
    }
  }
}

// Routing key of the raw product x for key block j: the score
// scale·x + cov_weight·M_j (+inf for the sink), mapped by order_key.
__device__ __forceinline__ unsigned long long route_key(const RouteArgs& a, long bh, double x, int j) {
  double sc = a.scale * x;
  if (a.cov_weight != 0.0) sc = sc + a.cov_weight * a.mnorm[bh * a.n + j];
  if (j == a.sink_block) sc = __builtin_huge_val();
  return order_key(sc);
}

// Wave-wide OR / AND of a 32-bit value through DPP (within rows of 16 lanes)
// and the four rows' first lanes; the result is uniform.
__device__ __forceinline__ uint32_t row16_or(uint32_t x) {
  x |= (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false);   // quad_perm 1,0,3,2
  x |= (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false);   // quad_perm 2,3,0,1
  x |= (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x141, 0xF, 0xF, false);  // row_half_mirror
  x |= (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x140, 0xF, 0xF, false);  // row_mirror
  return x;
}
__device__ __forceinline__ uint32_t wave_or32(uint32_t x) {
  x = row16_or(x);
  return (uint32_t)(__builtin_amdgcn_readlane((int)x, 0) | __builtin_amdgcn_readlane((int)x, 16) |
                    __builtin_amdgcn_readlane((int)x, 32) | __builtin_amdgcn_readlane((int)x, 48));
}
__device__ __forceinline__ uint32_t wave_and32(uint32_t x) { return ~wave_or32(~x); }

// Wave-wide sum of a 32-bit count through the same DPP steps: after each step
// every lane holds the sum over twice as many lanes of its row of 16 (quads,
// then half rows, then rows, each joined with its mirror image); the four rows'
// sums are then added on the scalar side. The result is uniform.
__device__ __forceinline__ int wave_sum32(int x) {
  x += __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);   // quad_perm 1,0,3,2
  x += __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);   // quad_perm 2,3,0,1
  x += __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, false);  // row_half_mirror
  x += __builtin_amdgcn_mov_dpp(x, 0x140, 0xF, 0xF, false);  // row_mirror
  return __builtin_amdgcn_readlane(x, 0) + __builtin_amdgcn_readlane(x, 16) +
         __builtin_amdgcn_readlane(x, 32) + __builtin_amdgcn_readlane(x, 48);
}

// MSB-first binary radix select over one wavefront's 32-bit keys (key[s] in
// lane j % 64, slot j / 64), counting with wave-wide sums. cand (bit s: slot s of
// this lane) holds the candidates, ncand of them, of which the kk largest are
// wanted. Each bit in which the candidates differ splits them: if at least kk
// have it set, the rest drop out; otherwise all that have it are taken (sel)
// and the search goes on among the others. On return either ncand == kk (every
// candidate left is taken) or the candidates left are equal in all 32 bits.
template <int KPL>
__device__ __forceinline__ void ballot_select(const uint32_t (&key)[KPL], uint32_t& cand, uint32_t& sel,
                                              int& kk, int& ncand) {
  uint32_t vor = 0u, vand = ~0u;
#pragma unroll
  for (int s = 0; s < KPL; ++s)
    if ((cand >> s) & 1u) {
      vor |= key[s];
      vand &= key[s];
    }
  uint32_t diff = wave_or32(vor) & ~wave_and32(vand);
  while (diff != 0u && ncand > kk) {
    const int b = 31 - __clz(diff);
    diff &= ~(1u << b);
    // the candidates with bit b set, gathered into one word per lane and
    // counted with a single wave-wide sum
    uint32_t ones = 0u;
#pragma unroll
    for (int s = 0; s < KPL; ++s) ones |= ((key[s] >> b) & 1u) << s;
    ones &= cand;
    const int cnt1 = wave_sum32(__popc(ones));
    if (cnt1 >= kk) {
      cand = ones;
      ncand = cnt1;
    } else {
      sel |= ones;
      cand &= ~ones;
      kk -= cnt1;
      ncand -= cnt1;
    }
  }
}

// Phase 2 for query block i (row il of the workgroup): selection and output.
// hrow: the row's upper key halves in LDS (this wavefront's alone from now on).
template <int D, int KPL>
__device__ __forceinline__ void route_row(const RouteArgs& a, long bh, int i, int il, uint32_t* hrow,
                                          const double* qb, const double* kb, int i0, int lane) {
  const int n = a.n, k = a.topk;
  int32_t* out = a.idx + ((size_t)bh * n + i) * k;
  uint32_t key[KPL];
  uint32_t cand = 0u, sel = 0u;
#pragma unroll
  for (int s = 0; s < KPL; ++s) {
    const int j = 64 * s + lane;
    key[s] = j < n ? hrow[j] : 0u;
    cand |= (j < n ? 1u : 0u) << s;
  }
  int kk = k, ncand = n;
  ballot_select<KPL>(key, cand, sel, kk, ncand);
  if (ncand > kk) {
    // The k-th place falls inside a run of keys equal in their upper halves,
    // and only part of the run is taken: the run's lower halves, from products
    // formed again (same code, same bits), decide within it.
    const int g = lane >> 4, c = lane & 15, g0 = il & 3, r0 = il >> 2;
    f64x4 A[D / 16];
    const double* pa = qb + (size_t)min(i0 + c, n - 1) * D + 4 * g;
#pragma unroll
    for (int ch = 0; ch < D / 16; ++ch) A[ch] = *reinterpret_cast<const f64x4*>(pa + 16 * ch);
    uint32_t smask = 0u;  // slots holding part of the run (uniform)
#pragma unroll
    for (int s = 0; s < KPL; ++s)
      if (__ballot((cand >> s) & 1u) != 0ull) smask |= 1u << s;
    while (smask != 0u) {
      const int s = __builtin_ctz(smask);
      smask &= smask - 1u;
      f64x4 acc[4];
      route_dots<D>(A, kb, 64 * s, n, g, c, acc);
      double x = 0.0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const double v = r0 == 0 ? acc[u][0] : r0 == 1 ? acc[u][1] : r0 == 2 ? acc[u][2] : acc[u][3];
        const double y = __shfl(v, 16 * g0 + c);  // row il, key block 64s + 16u + (lane & 15)
        if ((lane >> 4) == u) x = y;
      }
      const int j = 64 * s + lane;
      if (j < n) hrow[j] = (uint32_t)route_key(a, bh, x, j);
    }
#pragma unroll
    for (int s = 0; s < KPL; ++s) key[s] = ((cand >> s) & 1u) ? hrow[64 * s + lane] : 0u;
    ballot_select<KPL>(key, cand, sel, kk, ncand);
  }
  // the taken keys and, of the candidates left (equal in all 64 bits, or all
  // taken), the kk lowest-index ones, ascending
  const unsigned long long lt = (1ull << lane) - 1ull;
  int eq_seen = 0, pos = 0;
#pragma unroll
  for (int s = 0; s < KPL; ++s) {
    const bool above = (sel >> s) & 1u, eq = (cand >> s) & 1u;
    const unsigned long long beq = __ballot(eq);
    const bool take = above || (eq && eq_seen + __popcll(beq & lt) < kk);
    const unsigned long long bt = __ballot(take);
    const int at = pos + __popcll(bt & lt);
    if (take && at < k) out[at] = 64 * s + lane;  // exactly k are taken; the bound only guards the row
    pos += __popcll(bt);
    eq_seen += __popcll(beq);
  }
}

// Phase 1 for the 16 query blocks from i0 of head bh: NW wavefronts (this one
// is number w) share out the units of 32 key blocks; the upper key halves go
// to hk, rows of `stride`.
template <int D, int NW>
__device__ __forceinline__ void route_scores(const RouteArgs& a, long bh, int i0, int w, int lane,
                                             uint32_t* hk, int stride) {
  const int n = a.n, g = lane >> 4, c = lane & 15;
  const double* qb = a.qbar + (size_t)bh * n * D;
  const double* kb = a.kbar + (size_t)bh * n * D;
  // rows past the end repeat the last query block (formed, never selected)
  f64x4 A[D / 16];
  const double* pa = qb + (size_t)min(i0 + c, n - 1) * D + 4 * g;
#pragma unroll
  for (int ch = 0; ch < D / 16; ++ch) A[ch] = *reinterpret_cast<const f64x4*>(pa + 16 * ch);
  const int nunit = (n + 31) >> 5;
  for (int un = w; un < nunit; un += NW) {
    f64x4 acc[2];
    route_dots<D, 2>(A, kb, 32 * un, n, g, c, acc);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int j = 32 * un + 16 * u + c;
      if (j < n) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          hk[(g + 4 * r) * stride + j] = (uint32_t)(route_key(a, bh, acc[u][r], j) >> 32);
      }
    }
  }
}

// One workgroup of NW wavefronts per tile of 16 query blocks; rows of up to
// 64·KPL blocks, LDS rows of CAP keys; NW / 4 wavefronts per SIMD and two
// workgroups per CU.
template <int D, int NW, int KPL, int CAP>
__global__ __launch_bounds__(64 * NW, NW / 2) void k_route(RouteArgs a) {
  __shared__ uint32_t hk[kRouteRows * CAP];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  // Workgroups reach the eight XCDs in turn; each XCD takes consecutive row
  // tiles, so its L2 holds the k̄ of one or two heads at a time.
  long b = blockIdx.x;
  if ((a.total & 7) == 0) b = (b & 7) * (a.total >> 3) + (b >> 3);
  const long bh = b / a.nrt;
  const int i0 = (int)(b % a.nrt) * kRouteRows;
  const int n = a.n, k = a.topk;
  if (k >= n) {
    for (int il = wv; il < kRouteRows && i0 + il < n; il += NW) {
      int32_t* out = a.idx + ((size_t)bh * n + i0 + il) * k;
      for (int j = lane; j < n; j += 64) out[j] = j;
    }
    return;
  }
  const int stride = (n + 15) & ~15;
  route_scores<D, NW>(a, bh, i0, wv, lane, hk, stride);
  __syncthreads();
  const double* qb = a.qbar + (size_t)bh * n * D;
  const double* kb = a.kbar + (size_t)bh * n * D;
  for (int il = wv; il < kRouteRows && i0 + il < n; il += NW)
    route_row<D, KPL>(a, bh, i0 + il, il, hk + il * stride, qb, kb, i0, lane);
}

// MFMA products per wavefront of k_scores_mfma (rows x columns of 16 x 16).
// 4 x 4 needs ~300 registers (one wavefront per SIMD) and still beats 4 x 2
// and 2 x 2, which fit two and four: fewer operand loads per product count
// for more than occupancy here.
constexpr int kScoreTR = 4, kScoreTC = 4;

// Rows longer than kRouteMaxBlocks only (n > 1280).
hipError_t launch_scores(int D, const ScoreArgs& a, long bh, hipStream_t s) {
  if (a.n <= kRouteMaxBlocks) return hipErrorInvalidValue;
  constexpr int TR = kScoreTR, TC = kScoreTC;
  dim3 grid((unsigned)((a.n + 32 * TC - 1) / (32 * TC)), (unsigned)((a.n + 32 * TR - 1) / (32 * TR)),
            (unsigned)bh);
  if (D == 64) hipLaunchKernelGGL((k_scores_mfma<64, TR, TC>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((k_scores_mfma<128, TR, TC>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_topk(const TopkArgs& a, long rows, hipStream_t s) {
  const int slots = (a.n + 63) / 64;
  if (slots > 32) {
    const size_t lds = (size_t)a.n * sizeof(unsigned long long);
    hipLaunchKernelGGL(k_topk, dim3((unsigned)rows), dim3(256), lds, s, a);
    return hipGetLastError();
  }
  // rows of 1281 to 2048 blocks: 21 to 32 register slots
  if (a.n <= kRouteMaxBlocks) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((rows + 3) / 4));
  switch ((slots + 3) / 4) {
    case 6: hipLaunchKernelGGL(k_topk_wave<24>, grid, dim3(256), 0, s, a, rows); break;
    case 7: hipLaunchKernelGGL(k_topk_wave<28>, grid, dim3(256), 0, s, a, rows); break;
    default: hipLaunchKernelGGL(k_topk_wave<32>, grid, dim3(256), 0, s, a, rows); break;
  }
  return hipGetLastError();
}

template <int D>
static hipError_t launch_route_d(const RouteArgs& a, hipStream_t s) {
  const int slots = (a.n + 63) / 64, kpl = (slots + 3) / 4 * 4;
  const dim3 grid((unsigned)a.total);
  switch (kpl) {
    case 4: hipLaunchKernelGGL((k_route<D, 8, 4, 256>), grid, dim3(512), 0, s, a); break;
    case 8: hipLaunchKernelGGL((k_route<D, 8, 8, 512>), grid, dim3(512), 0, s, a); break;
    case 12: hipLaunchKernelGGL((k_route<D, 8, 12, 768>), grid, dim3(512), 0, s, a); break;
    case 16: hipLaunchKernelGGL((k_route<D, 8, 16, 1024>), grid, dim3(512), 0, s, a); break;
    default: hipLaunchKernelGGL((k_route<D, 8, 20, kRouteMaxBlocks>), grid, dim3(512), 0, s, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_route(int D, const RouteArgs& a, hipStream_t s) {
  if (a.n < 1 || a.n > kRouteMaxBlocks) return hipErrorInvalidValue;
  return D == 64 ? launch_route_d<64>(a, s) : launch_route_d<128>(a, s);
}

}  // namespace pisa
