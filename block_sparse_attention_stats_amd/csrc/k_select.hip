// Per-query-block top-k routing (gist.science technical summary of arXiv
// 2602.01077, section 2 "Covariance-Aware Routing"; the authors' README,
// "Attention sink for MMDiT").
//
// Scores: S_ij = scale * q̄_i·k̄_j + cov_weight * M_j in fp64 over (query block,
//   key block) tiles (n x n x D per head: small next to the fused pass); the
//   sink column gets +infinity. k_scores_mfma (n >= 512) on the fp64 matrix
//   cores; k_scores (shorter rows) a register-tiled fp64 GEMM through LDS.
// Top-k of a row: the k-th largest key T is narrowed down by an MSB-first
//   radix select over order-preserving 64-bit keys, stopping early once the
//   bucket that holds it is to be taken whole; then every key above T and the
//   lowest-index keys equal to it are taken, and the indices emitted ascending.
//   k_topk_wave (rows of up to 2048 blocks): one wavefront per row, its keys in
//   registers; each pass's 8-bit digit starts at the highest bit in which the
//   remaining candidates still differ, so no pass is spent on the sign and
//   exponent bits they share. k_topk (longer rows): one workgroup per row, the
//   keys in LDS, fixed 8-bit digits. Both return the same set.
#include "pisa_dev.h"
#include "pisa_internal.h"

namespace pisa {

// k_scores tile: TM x TM (query block, key block) pairs per workgroup, each of
// the 256 threads owning an (TM/16) x (TM/16) block of them (TM = 64 for the
// rows it serves, n < 512).
template <int D, int TM>
__global__ __launch_bounds__(256) void k_scores(ScoreArgs a) {
  // Rows ty + 16x, columns tx + 16y. The dot products run over d in order, one
  // fp64 FMA per term. The next chunk of q̄ / k̄ is read into registers while
  // the current one is consumed from LDS.
  constexpr int KC = 8, R = TM / 16, PER = TM * KC / 256;
  __shared__ double As[KC][TM + 1], Bs[KC][TM + 1];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const long bh = blockIdx.z;
  const int i0 = blockIdx.y * TM, j0 = blockIdx.x * TM;
  const double* qb = a.qbar + (size_t)bh * a.n * D;
  const double* kb = a.kbar + (size_t)bh * a.n * D;
  double acc[R][R];
#pragma unroll
  for (int x = 0; x < R; ++x)
#pragma unroll
    for (int y = 0; y < R; ++y) acc[x][y] = 0.0;
  double pa[PER], pb[PER];
  auto fetch = [&](int d0) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int x = tid + 256 * u, row = x / KC, dd = x % KC;
      pa[u] = (i0 + row < a.n) ? qb[(size_t)(i0 + row) * D + d0 + dd] : 0.0;
      pb[u] = (j0 + row < a.n) ? kb[(size_t)(j0 + row) * D + d0 + dd] : 0.0;
    }
  };
  fetch(0);
  for (int d0 = 0; d0 < D; d0 += KC) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int x = tid + 256 * u, row = x / KC, dd = x % KC;
      As[dd][row] = pa[u];
      Bs[dd][row] = pb[u];
    }
    __syncthreads();
    if (d0 + KC < D) fetch(d0 + KC);
#pragma unroll
    for (int dd = 0; dd < KC; ++dd) {
      double av[R], bv[R];
#pragma unroll
      for (int x = 0; x < R; ++x) av[x] = As[dd][ty + 16 * x];
#pragma unroll
      for (int y = 0; y < R; ++y) bv[y] = Bs[dd][tx + 16 * y];
#pragma unroll
      for (int x = 0; x < R; ++x)
#pragma unroll
        for (int y = 0; y < R; ++y) acc[x][y] = fma(av[x], bv[y], acc[x][y]);
    }
    __syncthreads();
  }
  double* out = a.scores + (size_t)bh * a.n * a.n;
#pragma unroll
  for (int y = 0; y < R; ++y) {
    const int j = j0 + tx + 16 * y;
    if (j >= a.n) continue;
    const double cov = a.cov_weight != 0.0 ? a.cov_weight * a.mnorm[bh * a.n + j] : 0.0;
#pragma unroll
    for (int x = 0; x < R; ++x) {
      const int i = i0 + ty + 16 * x;
      if (i >= a.n) continue;
      double sc = a.scale * acc[x][y];
      if (a.cov_weight != 0.0) sc = sc + cov;
      if (j == a.sink_block) sc = __builtin_huge_val();
      out[(size_t)i * a.n + j] = sc;
    }
  }
}

typedef double f64x4 __attribute__((ext_vector_type(4)));

// k_scores_mfma: the same scores on the fp64 matrix cores, for n >= 512.
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

// MFMA products per wavefront of k_scores_mfma (rows x columns of 16 x 16).
// 4 x 4 needs ~300 registers (one wavefront per SIMD) and still beats 4 x 2
// and 2 x 2, which fit two and four: fewer operand loads per product count
// for more than occupancy here.
constexpr int kScoreTR = 4, kScoreTC = 4;

hipError_t launch_scores(int D, const ScoreArgs& a, long bh, hipStream_t s) {
  if (a.n >= 512) {
    constexpr int TR = kScoreTR, TC = kScoreTC;
    dim3 grid((unsigned)((a.n + 32 * TC - 1) / (32 * TC)), (unsigned)((a.n + 32 * TR - 1) / (32 * TR)),
              (unsigned)bh);
    if (D == 64) hipLaunchKernelGGL((k_scores_mfma<64, TR, TC>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_scores_mfma<128, TR, TC>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
  }
  const unsigned t = (unsigned)((a.n + 63) / 64);
  dim3 grid(t, t, (unsigned)bh);
  if (D == 64) hipLaunchKernelGGL((k_scores<64, 64>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((k_scores<128, 64>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_topk(const TopkArgs& a, long rows, hipStream_t s) {
  const int slots = (a.n + 63) / 64;
  if (slots > 32) {
    const size_t lds = (size_t)a.n * sizeof(unsigned long long);
    hipLaunchKernelGGL(k_topk, dim3((unsigned)rows), dim3(256), lds, s, a);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((rows + 3) / 4));
  switch ((slots + 3) / 4) {
    case 1: hipLaunchKernelGGL(k_topk_wave<4>, grid, dim3(256), 0, s, a, rows); break;
    case 2: hipLaunchKernelGGL(k_topk_wave<8>, grid, dim3(256), 0, s, a, rows); break;
    case 3: hipLaunchKernelGGL(k_topk_wave<12>, grid, dim3(256), 0, s, a, rows); break;
    case 4: hipLaunchKernelGGL(k_topk_wave<16>, grid, dim3(256), 0, s, a, rows); break;
    case 5: hipLaunchKernelGGL(k_topk_wave<20>, grid, dim3(256), 0, s, a, rows); break;
    case 6: hipLaunchKernelGGL(k_topk_wave<24>, grid, dim3(256), 0, s, a, rows); break;
    case 7: hipLaunchKernelGGL(k_topk_wave<28>, grid, dim3(256), 0, s, a, rows); break;
    default: hipLaunchKernelGGL(k_topk_wave<32>, grid, dim3(256), 0, s, a, rows); break;
  }
  return hipGetLastError();
}

}  // namespace pisa
