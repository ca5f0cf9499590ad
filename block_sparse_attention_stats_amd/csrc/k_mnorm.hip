// Spectral covariance norm of every block (gist.science technical summary of
// arXiv 2602.01077, section 2 "Covariance-Aware Routing": M_j = ||H_j − H̄||_2,
// the largest singular value of block j's first-order matrix minus the mean).
//
// A fixed-step fp64 method whose accuracy does not depend on the gap between
// the largest singular values (as a power iteration's would). One 256-thread
// workgroup per block, the D x D Gram matrix held in registers throughout
// (thread (ta, tb) of a 16 x 16 grid owns rows ta*TS .. ta*TS+TS-1 and columns
// tb*TS .. tb*TS+TS-1, TS = D/16):
//   1. A = H_j − H̄ in chunks of 8 rows: the block's Σ_t k_t[r] v_t[e] from its
//      keys and values (products of bf16 or fp32 inputs are exact in fp64;
//      each thread keeps D/32 independent sums), minus k̄_j[r] ΣV_j[e] and
//      H̄[r][e]; each chunk goes through LDS and its rows' outer products are
//      added to the Gram matrix AᵀA;
//   2. the Gram matrix is reduced to tridiagonal form by D − 2 Householder
//      reflections applied from both sides (the symmetric tridiagonal
//      reduction). Step k maps column k below the diagonal to s·e1 with
//      P = I − β v vᵀ and updates the trailing block B ← B − v wᵀ − w vᵀ,
//      w = p − (β/2)(pᵀv) v, p = β B v: the column goes through LDS, B v is
//      summed over the 16 threads of a row group with DPP moves, and the
//      rank-two update is applied in registers;
//   3. its largest eigenvalue is bracketed between the largest diagonal entry
//      and the Gershgorin bound and narrowed by 8 rounds of 256-point
//      multisection, each point's Sturm count (eigenvalues below it) taken by
//      one thread; M_j = sqrt of the eigenvalue.
// The reduction is backward stable, so the eigenvalue is exact to about
// D^1.5 · 2^-53 relative, far inside the routing tie band.
#include "pisa_dev.h"
#include "pisa_internal.h"

namespace pisa {

namespace {

template <typename T, int D>
struct SpecShared {
  T kt[128][D];                       // the block's keys and values as read
  T vt[128][D];
  double arow[8][D];                  // a chunk of rows of A, added to the Gram matrix
  double col[2][D];                   // column k of the trailing block (by the parity of k)
  double wv[D];                       // w of the current reflection
  double dg[D], od[D];                // tridiagonal result: diagonal, off-diagonal
  double red[4];
  unsigned long long ballot[4];
};

// Moves a double between lanes with one DPP pattern (two 32-bit moves).
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
  const long long b = __double_as_longlong(x);
  const int lo = __builtin_amdgcn_mov_dpp((int)b, CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_mov_dpp((int)(b >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

// Sum over the 16 lanes of a DPP row, every lane receiving it: pairs (lane
// xor 1), quads (xor 2), the two halves of each 8-lane half row mirrored, then
// the two halves of the row mirrored. Each step adds a disjoint partner set.
__device__ __forceinline__ double row_sum16(double x) {
  x += dpp_f64<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_f64<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_f64<0x141>(x);  // row_half_mirror
  x += dpp_f64<0x140>(x);  // row_mirror
  return x;
}

template <typename T, int D, bool SEG>
__global__ __launch_bounds__(256, 2) void k_mnorm_spectral(StatsArgs a) {
  using O = Op<T>;
  constexpr int KW = Geo<T, D>::KW, CPR = Geo<T, D>::CPR;
  constexpr int TS = D / 16;
  __shared__ SpecShared<T, D> sh;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const long bh = blockIdx.x / a.n;
  const int j = (int)(blockIdx.x % a.n);
  const int nj = min(a.blk, a.L - j * a.blk);
  const long bat = bh / a.H, hd = bh % a.H;
  const size_t head_off = (size_t)bat * a.stride_b + (size_t)hd * a.stride_h;
  const size_t head_off1 = (size_t)bat * a.stride1_b + (size_t)hd * a.stride1_h;

  // ---- 1. the block's keys and values into LDS
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
    *(uint4*)&sh.kt[t][c * KW] = *(const uint4*)(ks + off + c * 16);
    *(uint4*)&sh.vt[t][c * KW] = *(const uint4*)(vs + off + c * 16);
  }
  __syncthreads();

  // A in chunks of 8 rows through LDS; the Gram matrix in registers. Thread
  // (row rr = tid / 32, columns 4·(tid % 32) .. +3) forms 4 entries of a chunk
  // row as 4 independent fp64 sums over the block's tokens.
  const int ta = tid >> 4, tb = tid & 15;
  double g[TS][TS];
#pragma unroll
  for (int x = 0; x < TS; ++x)
#pragma unroll
    for (int y = 0; y < TS; ++y) g[x][y] = 0.0;
  const double* kb = a.kbar + ((size_t)bh * a.n + j) * D;
  const double* vb = a.vsum + ((size_t)bh * a.n + j) * D;
  const double* hb = a.hbar + (size_t)bh * D * D;
  constexpr int CW = D / 32;  // columns per thread in a chunk row
  for (int r0 = 0; r0 < D; r0 += 8) {
    const int r = r0 + (tid >> 5), e0 = CW * (tid & 31);
    double acc[CW];
#pragma unroll
    for (int c = 0; c < CW; ++c) acc[c] = 0.0;
    for (int t = 0; t < nj; ++t) {
      const double kv = (double)O::to_f32(sh.kt[t][r]);
#pragma unroll
      for (int c = 0; c < CW; ++c) acc[c] = fma(kv, (double)O::to_f32(sh.vt[t][e0 + c]), acc[c]);
    }
    const double kr = kb[r];
#pragma unroll
    for (int c = 0; c < CW; ++c) sh.arow[tid >> 5][e0 + c] = (acc[c] - kr * vb[e0 + c]) - hb[r * D + e0 + c];
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      double ax[TS], ay[TS];
#pragma unroll
      for (int x = 0; x < TS; ++x) ax[x] = sh.arow[q][ta * TS + x];
#pragma unroll
      for (int y = 0; y < TS; ++y) ay[y] = sh.arow[q][tb * TS + y];
#pragma unroll
      for (int x = 0; x < TS; ++x)
#pragma unroll
        for (int y = 0; y < TS; ++y) g[x][y] = fma(ax[x], ay[y], g[x][y]);
    }
    __syncthreads();
  }

  // ---- 2. symmetric tridiagonal reduction, the matrix in registers. Column
  // index k = kb·TS + y with y unrolled, so the owners' register is static.
  // Entries outside the trailing block see v = w = 0 and stay as they are.
  for (int kq = 0; kq < D / TS; ++kq) {
#pragma unroll
    for (int y = 0; y < TS; ++y) {
      const int k = kq * TS + y;
      if (k <= D - 3) {
        const int b0 = k + 1;
        // two column buffers: a step that skips its reflection has no barrier
        // after its reads, so the next step writes the other buffer
        double* colk = sh.col[k & 1];
        if (tb == kq) {
#pragma unroll
          for (int x = 0; x < TS; ++x)
            if (ta * TS + x >= b0) colk[ta * TS + x] = g[x][y];
          if (ta == kq) sh.dg[k] = g[y][y];
        }
        __syncthreads();
        // every wavefront forms the same reflector from the column
        double t2 = 0.0;
#pragma unroll
        for (int h = 0; h < D; h += 64) {
          const int r = h + lane;
          const double xv = (r > b0 && r < D) ? colk[r] : 0.0;
          t2 = fma(xv, xv, t2);
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) t2 += __shfl_xor(t2, o);
        const double x0 = colk[b0];
        if (t2 == 0.0) {  // column already reduced: no reflection (uniform branch)
          if (tid == 0) sh.od[k] = x0;
          continue;
        }
        const double alpha = sqrt(fma(x0, x0, t2));
        const double s = x0 >= 0.0 ? -alpha : alpha;
        const double v0 = x0 - s;
        const double beta = 2.0 / fma(v0, v0, t2);
        if (tid == 0) sh.od[k] = s;
        double vr[TS], vc[TS];
#pragma unroll
        for (int x = 0; x < TS; ++x) {
          const int r = ta * TS + x, c = tb * TS + x;
          vr[x] = r == b0 ? v0 : (r > b0 ? colk[r] : 0.0);
          vc[x] = c == b0 ? v0 : (c > b0 ? colk[c] : 0.0);
        }
        // p = β B v for this thread's rows: partial over its columns, then
        // summed over the 16 threads of the row group (consecutive lanes)
        double p[TS];
#pragma unroll
        for (int x = 0; x < TS; ++x) {
          double acc = 0.0;
#pragma unroll
          for (int yy = 0; yy < TS; ++yy) acc = fma(g[x][yy], vc[yy], acc);
          p[x] = acc;
        }
#pragma unroll
        for (int x = 0; x < TS; ++x) p[x] = row_sum16(p[x]);
        double ptv = 0.0;
#pragma unroll
        for (int x = 0; x < TS; ++x) {
          p[x] *= beta;
          ptv = fma(p[x], vr[x], ptv);
        }
        // pᵀv: one term per row group (its lane tb = 0), then over the wavefronts
        ptv = tb == 0 ? ptv : 0.0;
        ptv += __shfl_xor(ptv, 16);
        ptv += __shfl_xor(ptv, 32);
        if (lane == 0) sh.red[wv] = ptv;
        double wr[TS];
        __syncthreads();
        const double kk = 0.5 * beta * ((sh.red[0] + sh.red[1]) + (sh.red[2] + sh.red[3]));
#pragma unroll
        for (int x = 0; x < TS; ++x) {
          const int r = ta * TS + x;
          wr[x] = r >= b0 ? fma(-kk, vr[x], p[x]) : 0.0;
          if (tb == 0) sh.wv[r] = wr[x];
        }
        __syncthreads();
#pragma unroll
        for (int yy = 0; yy < TS; ++yy) {
          const double wc = sh.wv[tb * TS + yy];
#pragma unroll
          for (int x = 0; x < TS; ++x) g[x][yy] -= fma(vr[x], wc, wr[x] * vc[yy]);
        }
      }
    }
  }
  {
    constexpr int q2 = (D - 2) / TS, y2 = (D - 2) % TS, q1 = (D - 1) / TS, y1 = (D - 1) % TS;
    if (ta == q2 && tb == q2) sh.dg[D - 2] = g[y2][y2];
    if (ta == q1 && tb == q1) sh.dg[D - 1] = g[y1][y1];
    if (ta == q1 && tb == q2) sh.od[D - 2] = g[y1][y2];
    if (tid == 0) sh.od[D - 1] = 0.0;
  }
  __syncthreads();

  // ---- 3. the largest eigenvalue of the tridiagonal matrix: 8 rounds of
  // 256-point multisection, one point per thread
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
  for (int round = 0; round < 8 && hi > lo; ++round) {
    const double x = lo + (hi - lo) * (double)(tid + 1) / 257.0;
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
    // the largest eigenvalue lies below x exactly where every eigenvalue does;
    // the first such point over the four wavefronts closes the bracket
    const unsigned long long above = __ballot(cnt == D);
    if (lane == 0) sh.ballot[wv] = above;
    __syncthreads();
    int first = 256;
#pragma unroll
    for (int w = 3; w >= 0; --w)
      if (sh.ballot[w]) first = 64 * w + __ffsll(sh.ballot[w]) - 1;
    __syncthreads();  // ballots read before the next round writes them
    const double nhi = first < 256 ? lo + (hi - lo) * (double)(first + 1) / 257.0 : hi;
    const double nlo = first > 0 ? lo + (hi - lo) * (double)first / 257.0 : lo;
    hi = nhi;
    lo = nlo;
  }
  if (tid == 0) a.mnorm[bh * a.n + j] = sqrt(fmax(hi, 0.0));
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
