// Spectral covariance norm of every block (gist.science technical summary of
// arXiv 2602.01077, section 2 "Covariance-Aware Routing": M_j = ||H_j − H̄||_2,
// the largest singular value of block j's first-order matrix minus the mean).
//
// A fixed-step fp64 method whose accuracy does not depend on the gap between
// the largest singular values (as a power iteration's would). One workgroup
// per block:
//   1. A = H_j − H̄ row by row in fp64: the block's Σ_t k_t[r] v_t[e] from its
//      keys and values (products of bf16 or fp32 inputs are exact in fp64),
//      minus k̄_j[r] ΣV_j[e] and H̄[r][e]; each row's outer product is added to
//      the Gram matrix AᵀA, held in registers (an 8 x 8 tile per thread);
//   2. the Gram matrix goes to LDS and is reduced to tridiagonal form by D − 2
//      Householder reflections applied from both sides (the symmetric
//      tridiagonal reduction), all in fp64;
//   3. its largest eigenvalue is bracketed between the largest diagonal entry
//      and the Gershgorin bound and narrowed by 12 rounds of 64-point
//      multisection, each point's Sturm count (eigenvalues below it) taken by
//      one lane; M_j = sqrt of the eigenvalue.
// The reduction is backward stable, so the eigenvalue is exact to about
// D^1.5 · 2^-53 relative, far inside the routing tie band.
#include "pisa_dev.h"
#include "pisa_internal.h"

namespace pisa {

namespace {

template <int D>
struct SpecShared {
  static constexpr int RP = 256 / D;  // rows of A formed per pass
  union {
    struct {
      float kt[128][D];     // the block's keys and values, widened exactly to fp32
      float vt[128][D];
      double arow[RP][D];   // rows of A being added to the Gram matrix
    } p1;
    double g[D][D + 1];     // Gram matrix (odd row pitch: column reads spread over banks)
  } u;
  double v[D], p[D], w[D];  // Householder vector, B·v, update vector
  double dg[D], od[D];      // tridiagonal result: diagonal, off-diagonal
  double red[4];
};

// Sum over the 256 threads (every thread gets the total).
__device__ __forceinline__ double block_sum(double x, double* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  const int wv = threadIdx.x >> 6;
  __syncthreads();  // red free
  if ((threadIdx.x & 63) == 0) red[wv] = x;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

template <typename T, int D, bool SEG>
__global__ __launch_bounds__(256, 1) void k_mnorm_spectral(StatsArgs a) {
  using O = Op<T>;
  constexpr int KW = Geo<T, D>::KW, CPR = Geo<T, D>::CPR;
  constexpr int RP = SpecShared<D>::RP, TS = D / 16;
  __shared__ SpecShared<D> sh;
  const int tid = threadIdx.x;
  const long bh = blockIdx.x / a.n;
  const int j = (int)(blockIdx.x % a.n);
  const int nj = min(a.blk, a.L - j * a.blk);
  const long bat = bh / a.H, hd = bh % a.H;
  const size_t head_off = (size_t)bat * a.stride_b + (size_t)hd * a.stride_h;
  const size_t head_off1 = (size_t)bat * a.stride1_b + (size_t)hd * a.stride1_h;

  // ---- 1. the block's keys and values into LDS as fp32
  for (int x = tid; x < nj * CPR; x += 256) {
    const int t = x / CPR, c = x % CPR;
    const int grow = j * a.blk + t;
    size_t off;
    const uint8_t *ks, *vs;
    if (!SEG || grow < a.L0) {
      off = head_off + (size_t)grow * a.stride_l;
      ks = a.k;
      vs = a.v;
    } else {
      off = head_off1 + (size_t)(grow - a.L0) * a.stride1_l;
      ks = a.k1;
      vs = a.v1;
    }
    const uint4 kc = *(const uint4*)(ks + off + c * 16);
    const uint4 vc = *(const uint4*)(vs + off + c * 16);
    const T* kx = (const T*)&kc;
    const T* vx = (const T*)&vc;
#pragma unroll
    for (int e = 0; e < KW; ++e) {
      sh.u.p1.kt[t][c * KW + e] = O::to_f32(kx[e]);
      sh.u.p1.vt[t][c * KW + e] = O::to_f32(vx[e]);
    }
  }
  __syncthreads();

  // A row by row; the Gram matrix in registers: thread (ta, tb) owns rows
  // ta*TS .. ta*TS+TS-1 and columns tb*TS .. tb*TS+TS-1
  const int ta = tid >> 4, tb = tid & 15;
  double gacc[TS][TS];
#pragma unroll
  for (int x = 0; x < TS; ++x)
#pragma unroll
    for (int y = 0; y < TS; ++y) gacc[x][y] = 0.0;
  const double* kb = a.kbar + ((size_t)bh * a.n + j) * D;
  const double* vb = a.vsum + ((size_t)bh * a.n + j) * D;
  const double* hb = a.hbar + (size_t)bh * D * D;
  for (int r0 = 0; r0 < D; r0 += RP) {
    const int rr = tid / D, r = r0 + rr, e = tid % D;
    double acc = 0.0;
    for (int t = 0; t < nj; ++t) acc = fma((double)sh.u.p1.kt[t][r], (double)sh.u.p1.vt[t][e], acc);
    sh.u.p1.arow[rr][e] = (acc - kb[r] * vb[e]) - hb[r * D + e];
    __syncthreads();
#pragma unroll
    for (int q = 0; q < RP; ++q) {
      double ax[TS], ay[TS];
#pragma unroll
      for (int x = 0; x < TS; ++x) ax[x] = sh.u.p1.arow[q][ta * TS + x];
#pragma unroll
      for (int y = 0; y < TS; ++y) ay[y] = sh.u.p1.arow[q][tb * TS + y];
#pragma unroll
      for (int x = 0; x < TS; ++x)
#pragma unroll
        for (int y = 0; y < TS; ++y) gacc[x][y] = fma(ax[x], ay[y], gacc[x][y]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int x = 0; x < TS; ++x)
#pragma unroll
    for (int y = 0; y < TS; ++y) sh.u.g[ta * TS + x][tb * TS + y] = gacc[x][y];
  __syncthreads();

  // ---- 2. symmetric tridiagonal reduction: step k maps column k below the
  // diagonal to s·e1 with P = I − beta v vᵀ, v = x − s e1, and updates the
  // trailing block B ← P B P = B − v wᵀ − w vᵀ, w = p − (beta/2)(pᵀv) v, p = beta B v
  for (int k = 0; k < D - 2; ++k) {
    const int m = D - 1 - k, b0 = k + 1;
    const double xi = tid < m ? sh.u.g[b0 + tid][k] : 0.0;
    const double tail2 = block_sum(tid >= 1 && tid < m ? xi * xi : 0.0, sh.red);
    const double x0 = sh.u.g[b0][k];
    if (tail2 == 0.0) {  // column already reduced: no reflection (uniform branch)
      if (tid == 0) {
        sh.dg[k] = sh.u.g[k][k];
        sh.od[k] = x0;
      }
      continue;
    }
    const double alpha = sqrt(x0 * x0 + tail2);
    const double s = x0 >= 0.0 ? -alpha : alpha;
    const double v0 = x0 - s;
    const double beta = 2.0 / (v0 * v0 + tail2);
    if (tid < m) sh.v[tid] = tid == 0 ? v0 : xi;
    if (tid == 0) {
      sh.dg[k] = sh.u.g[k][k];
      sh.od[k] = s;
    }
    __syncthreads();
    // p = beta B v: two threads per row, each over half of the columns
    const int i = tid >> 1, half = tid & 1;
    double pi = 0.0;
    if (i < m) {
      const int jh = (m + 1) >> 1, j0 = half ? jh : 0, j1 = half ? m : jh;
      for (int jj = j0; jj < j1; ++jj) pi = fma(sh.u.g[b0 + i][b0 + jj], sh.v[jj], pi);
    }
    pi += __shfl_xor(pi, 1);
    pi *= beta;
    if (i < m && half == 0) sh.p[i] = pi;
    const double ptv = block_sum(i < m && half == 0 ? pi * sh.v[i] : 0.0, sh.red);
    const double kk = 0.5 * beta * ptv;
    if (tid < m) sh.w[tid] = sh.p[tid] - kk * sh.v[tid];
    __syncthreads();
    for (int x = tid; x < m * m; x += 256) {
      const int ii = x / m, jj = x - ii * m;
      sh.u.g[b0 + ii][b0 + jj] -= sh.v[ii] * sh.w[jj] + sh.w[ii] * sh.v[jj];
    }
    __syncthreads();
  }
  if (tid == 0) {
    sh.dg[D - 2] = sh.u.g[D - 2][D - 2];
    sh.dg[D - 1] = sh.u.g[D - 1][D - 1];
    sh.od[D - 2] = sh.u.g[D - 1][D - 2];
    sh.od[D - 1] = 0.0;
  }
  __syncthreads();

  // ---- 3. the largest eigenvalue of the tridiagonal matrix (wavefront 0)
  if (tid >= 64) return;
  const int lane = tid;
  double lo = 0.0, hi = 0.0, e2max = 0.0;  // the Gram matrix is positive semidefinite
  for (int x = lane; x < D; x += 64) {
    const double ol = x > 0 ? fabs(sh.od[x - 1]) : 0.0, orr = x < D - 1 ? fabs(sh.od[x]) : 0.0;
    lo = fmax(lo, sh.dg[x]);
    hi = fmax(hi, sh.dg[x] + ol + orr);
    e2max = fmax(e2max, orr * orr);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    lo = fmax(lo, __shfl_xor(lo, o));
    hi = fmax(hi, __shfl_xor(hi, o));
    e2max = fmax(e2max, __shfl_xor(e2max, o));
  }
  // smallest pivot magnitude kept by the Sturm recurrence
  const double pivmin = 2.2250738585072014e-308 * fmax(1.0, e2max);
  for (int round = 0; round < 12 && hi > lo; ++round) {
    const double x = lo + (hi - lo) * (double)(lane + 1) / 65.0;
    // eigenvalues below x: negative pivots of T − x I
    int cnt = 0;
    double q = sh.dg[0] - x;
    if (fabs(q) <= pivmin) q = -pivmin;
    cnt += q < 0.0;
    for (int t = 1; t < D; ++t) {
      q = (sh.dg[t] - x) - sh.od[t - 1] * sh.od[t - 1] / q;
      if (fabs(q) <= pivmin) q = -pivmin;
      cnt += q < 0.0;
    }
    // the largest eigenvalue lies below x exactly where every eigenvalue does
    const unsigned long long above = __ballot(cnt == D);
    const int first = above ? __ffsll(above) - 1 : 64;
    const double nhi = first < 64 ? __shfl(x, first) : hi;
    const double nlo = first > 0 ? __shfl(x, first - 1 < 63 ? first - 1 : 63) : lo;
    hi = nhi;
    lo = nlo;
  }
  if (lane == 0) a.mnorm[bh * a.n + j] = sqrt(fmax(hi, 0.0));
}

template <typename T, int D>
hipError_t launch_spec_t(const StatsArgs& a, long bh, hipStream_t s) {
  dim3 grid((unsigned)(bh * a.n));
  if (a.L0 < a.L)
    hipLaunchKernelGGL((k_mnorm_spectral<T, D, true>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((k_mnorm_spectral<T, D, false>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mnorm_spectral(int dtype, int D, const StatsArgs& a, long bh, hipStream_t s) {
  if (dtype == 1) return D == 64 ? launch_spec_t<bf16, 64>(a, bh, s) : launch_spec_t<bf16, 128>(a, bh, s);
  return D == 64 ? launch_spec_t<float, 64>(a, bh, s) : launch_spec_t<float, 128>(a, bh, s);
}

}  // namespace pisa
