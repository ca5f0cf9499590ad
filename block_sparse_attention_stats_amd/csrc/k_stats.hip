// Block statistics (PISA pre-computation; gist.science technical summary of
// arXiv 2602.01077, section 2 "Hardware Implementation" step 1, symbols of
// "Core Algorithm"): for every block j of a (batch, head)
//   q̄_j = mean of its query rows, k̄_j = mean of its keys, ΣV_j = Σ v,
//   H_j = Σ_n (k_n − k̄_j)ᵀ v_n, and H̄ = (1/n) Σ_j H_j;
// optionally M_j = ||H_j − H̄||_F ("Covariance-Aware Routing").
//
// One HBM-streaming pass: each workgroup walks a run of consecutive blocks of
// one head, staging 64-token sub-tiles of q, k, v through LDS (the next
// sub-tile is already loading while the current one is consumed). Per
// sub-tile it
//   * sums columns in fp64 (exact for bf16/fp32 inputs of one block),
//   * writes K and V in the operand order of the fused kernel (K-format and
//     V-format sub-tiles, see pisa_dev.h) so that kernel reads them with
//     whole-wavefront 1 KiB loads,
//   * accumulates G = Kᵀ V on MFMA (bf16 products are exact in fp32) and
//     subtracts k̄_j ⊗ ΣV_j once block j is complete, leaving Σ_j H_j of the
//     run in the accumulators; runs are summed in fp64 by k_hbar_reduce.
#include "pisa_dev.h"
#include "pisa_internal.h"

namespace pisa {

// SEG: the sequence is held in two tensors (rows from L0 on in q1, k1, v1).
// Without it the kernel never touches the second part, which keeps its state
// out of the registers the single-tensor case needs.
// Two transposed 8-byte LDS reads (gfx950's ds_read_b64_tr_b16) at p and
// eight rows further: the 16-bit MFMA operand of one column over two runs of
// four rows.
typedef short stats_v4s __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 col8_tr(const uint8_t* p, int pitch) {
  typedef __attribute__((address_space(3))) stats_v4s* lds_v4s;
  const stats_v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)p);
  const stats_v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(p + 8 * pitch));
  const uint2 x = __builtin_bit_cast(uint2, lo), y = __builtin_bit_cast(uint2, hi);
  return make_uint4(x.x, x.y, y.x, y.y);
}

template <typename T, int D, int MODE, bool SEG>
__global__ __launch_bounds__(256, 2) void k_block_stats(StatsArgs a) {
  using G = Geo<T, D>;
  using O = Op<T>;
  constexpr int KW = G::KW, ESZ = G::ESZ, CPR = G::CPR, NC = G::NC, DT = G::DT, CPK = G::CPK;
  constexpr int PITCH = G::ROW_BYTES + 16;  // padded LDS row: transposed reads spread over banks
  constexpr int NT = (MODE == kStatsFull) ? 3 : 2;
  constexpr int PER = 64 * CPR / 256;       // 16-byte chunks per thread per tensor per sub-tile
  constexpr int TW = DT / 2;                // G tiles per side per wave (2x2 waves)
  constexpr int KT = NT - 2, VT = NT - 1;   // LDS slots of k and v
  constexpr bool kDoG = (MODE != kStatsPackOnly);
  constexpr bool kDoPack = (MODE != kStatsMnorm);
  static_assert(PER >= 1 && TW >= 1, "shape");

  __shared__ __align__(16) uint8_t tile[NT][64 * PITCH];
  __shared__ float kbf[D], vsf[D];
  __shared__ double kbd[D], vsd[D];
  __shared__ double red[4];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, h = lane >> 5, l32 = lane & 31;
  const long bh = blockIdx.x / a.nch;
  const int ch = (int)(blockIdx.x % a.nch);
  const int j0 = ch * a.cb, j1 = min(a.n, j0 + a.cb);
  const int spb = a.blk / kSub;
  const int total_sub = (j1 - j0) * spb;
  const uint8_t *src[NT], *src1[NT];  // the two segments of the sequence
  if constexpr (MODE == kStatsFull) {
    src[0] = a.q; src[1] = a.k; src[2] = a.v;
    src1[0] = a.q1; src1[1] = a.k1; src1[2] = a.v1;
  } else {
    src[0] = a.k; src[1] = a.v;
    src1[0] = a.k1; src1[1] = a.v1;
  }
  const long bat = bh / a.H, hd = bh % a.H;
  const size_t head_off = (size_t)bat * a.stride_b + (size_t)hd * a.stride_h;
  const size_t head_off1 = (size_t)bat * a.stride1_b + (size_t)hd * a.stride1_h;

  // G tiles owned by this wave: rows d in tiles dt0.., columns e in tiles et0..
  const int dt0 = TW * (wv >> 1), et0 = TW * (wv & 1);
  f32x16 acc[TW][TW];
#pragma unroll
  for (int x = 0; x < TW; ++x)
#pragma unroll
    for (int y = 0; y < TW; ++y) acc[x][y] = f32x16{};

  double hb[TW][TW][16];  // H̄ entries of the owned tiles (mnorm pass)
  if constexpr (MODE == kStatsMnorm) {
#pragma unroll
    for (int x = 0; x < TW; ++x)
#pragma unroll
      for (int y = 0; y < TW; ++y)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int d = 32 * (dt0 + x) + vkey(r, h), e = 32 * (et0 + y) + l32;
          hb[x][y][r] = a.hbar[(bh * D + d) * D + e];
        }
  }

  // Column sums, in fp64: task p = ((tensor * CG + g) << 2) | rq sums the KW
  // columns of 16-byte group g over rows 16 rq .. 16 rq + 15 of each sub-tile
  // (p = tid, tid + 256). The four row quarters of a group are adjacent lanes
  // and are added together when the block is complete.
  constexpr int CG = D / KW, NTASK = 3 * CG * 4, NU = (NTASK + 255) / 256;
  double csum[NU][KW];
#pragma unroll
  for (int u = 0; u < NU; ++u)
#pragma unroll
    for (int e = 0; e < KW; ++e) csum[u][e] = 0.0;
  float kn2max = 0.0f;          // largest squared key norm seen by this thread's rows

  uint4 pre[NT][PER];
  auto load_sub = [&](int s) {
    const int j = j0 + s / spb, st = s % spb;
    const int r0 = j * a.blk + st * kSub;
    if constexpr (!SEG) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < PER; ++i) {
          const int x = tid + 256 * i, row = x / CPR, cc = x % CPR;
          const int grow = r0 + row;
          if (grow < a.L)
            pre[t][i] = *(const uint4*)(src[t] + head_off + (size_t)grow * a.stride_l + cc * 16);
          else
            pre[t][i] = make_uint4(0, 0, 0, 0);
        }
      return;
    }
    // The 64 rows lie in one part of the sequence unless they straddle L0:
    // then one base and stride (uniform) serve every load.
    const bool in0 = r0 + kSub <= a.L0, in1 = r0 >= a.L0;
    if (in0 || in1) {
      const size_t sl = in0 ? a.stride_l : a.stride1_l;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const uint8_t* base = in0 ? src[t] + head_off + (size_t)r0 * sl
                                  : src1[t] + head_off1 + (size_t)(r0 - a.L0) * sl;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
          const int x = tid + 256 * i, row = x / CPR, cc = x % CPR;
          pre[t][i] = r0 + row < a.L ? *(const uint4*)(base + (size_t)row * sl + cc * 16)
                                     : make_uint4(0, 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < PER; ++i) {
          const int x = tid + 256 * i, row = x / CPR, cc = x % CPR;
          const int grow = r0 + row;
          const uint8_t* p = grow < a.L0 ? src[t] + head_off + (size_t)grow * a.stride_l
                                         : src1[t] + head_off1 + (size_t)(grow - a.L0) * a.stride1_l;
          pre[t][i] = grow < a.L ? *(const uint4*)(p + cc * 16) : make_uint4(0, 0, 0, 0);
        }
    }
  };

  if (total_sub > 0) load_sub(0);
  for (int s = 0; s < total_sub; ++s) {
    const int j = j0 + s / spb, st = s % spb;
    __syncthreads();  // LDS free
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int x = tid + 256 * i, row = x / CPR, cc = x % CPR;
        *(uint4*)(&tile[t][row * PITCH + cc * 16]) = pre[t][i];
      }
    if constexpr (MODE == kStatsMnorm) {
      if (st == 0)
        for (int d = tid; d < D; d += 256) {
          kbd[d] = a.kbar[(bh * a.n + j) * D + d];
          vsd[d] = a.vsum[(bh * a.n + j) * D + d];
        }
    }
    __syncthreads();
    if (s + 1 < total_sub) load_sub(s + 1);

    // ---- fp64 column sums (q, k, v)
    if constexpr (MODE == kStatsFull) {
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int p = tid + 256 * u;
        if (p < NTASK) {
          const int t = (p >> 2) / CG, g = (p >> 2) % CG, rq = p & 3;
#pragma unroll 4
          for (int row = 16 * rq; row < 16 * rq + 16; ++row) {
            const uint4 c = *(const uint4*)(&tile[t][row * PITCH + g * 16]);
            const T* x = (const T*)&c;
#pragma unroll
            for (int e = 0; e < KW; ++e) csum[u][e] += (double)O::to_f32(x[e]);
          }
        }
      }
    }

    // ---- squared key norms (bound of the logits used by the fused pass)
    if constexpr (kDoPack) {
      const int row = tid >> 2, part = tid & 3;
      float ss = 0.0f;
      constexpr int NCH = D / 4 / KW;  // 16-byte chunks in a quarter row
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const uint4 ch16 = *(const uint4*)(&tile[KT][row * PITCH + (part * NCH + c) * 16]);
        const T* x = (const T*)&ch16;
#pragma unroll
        for (int e = 0; e < KW; ++e) {
          const float xf = O::to_f32(x[e]);
          ss = fmaf(xf, xf, ss);
        }
      }
      ss += __shfl_xor(ss, 1);
      ss += __shfl_xor(ss, 2);
      kn2max = fmaxf(kn2max, ss);
    }

    // ---- operand-ordered copies of K and V
    if constexpr (kDoPack) {
      const size_t sub_idx = ((size_t)bh * a.n + j) * spb + st;
      uint8_t* kdst = a.kp + sub_idx * G::SUB_BYTES;
      uint8_t* vdst = a.vp + sub_idx * G::SUB_BYTES;
#pragma unroll
      for (int i = 0; i < NC / 2; ++i) {
        const int u = tid + 256 * i, ul = u & 63, wc = u >> 6;
        const int w = wc / NC, c = wc % NC;
        const int kk = 32 * w + (ul & 31), d0 = 2 * KW * c + KW * (ul >> 5);
        *(uint4*)(kdst + (size_t)u * 16) = *(const uint4*)(&tile[KT][kk * PITCH + d0 * ESZ]);
      }
#pragma unroll
      for (int i = 0; i < DT * CPK / 2; ++i) {
        const int u = tid + 256 * i, ul = u & 63, ci = u >> 6;
        const int w = ci / (DT * CPK), rem = ci % (DT * CPK), dt = rem / CPK, c = rem % CPK;
        const int d = 32 * dt + (ul & 31), hh = ul >> 5;
        T vals[KW];
#pragma unroll
        for (int e = 0; e < KW; ++e)
          vals[e] = *(const T*)(&tile[VT][(32 * w + vkey(KW * c + e, hh)) * PITCH + d * ESZ]);
        *(uint4*)(vdst + (size_t)u * 16) = __builtin_bit_cast(uint4, vals);
      }
    }

    // ---- G += Kᵀ V on MFMA (contraction over the 64 tokens of the sub-tile)
    if constexpr (kDoG) {
#pragma unroll
      for (int w = 0; w < 2; ++w)
#pragma unroll
        for (int c = 0; c < CPK; ++c) {
          uint4 A[TW], B[TW];
#pragma unroll
          for (int x = 0; x < TW; ++x) {
            if constexpr (ESZ == 2) {
              // the eight key rows of vkey order are two runs of four: one
              // transposed read each (ds_read_b64_tr_b16; in each group of 16
              // lanes, lane i points at 4 elements of row r0 + i/4 from column
              // c0 + 4 (i % 4), and each lane receives its own column c0 + i)
              const int g = lane >> 4, i = lane & 15;
              const int row = 32 * w + 16 * c + 4 * h + (i >> 2);
              const int col = 16 * (g & 1) + 4 * (i & 3);
              A[x] = col8_tr(&tile[KT][row * PITCH + (32 * (dt0 + x) + col) * 2], PITCH);
              B[x] = col8_tr(&tile[VT][row * PITCH + (32 * (et0 + x) + col) * 2], PITCH);
            } else {
              T av[KW], bv[KW];
              const int dA = 32 * (dt0 + x) + l32, dB = 32 * (et0 + x) + l32;
#pragma unroll
              for (int e = 0; e < KW; ++e) {
                const int row = (32 * w + vkey(KW * c + e, h)) * PITCH;
                av[e] = *(const T*)(&tile[KT][row + dA * ESZ]);
                bv[e] = *(const T*)(&tile[VT][row + dB * ESZ]);
              }
              A[x] = __builtin_bit_cast(uint4, av);
              B[x] = __builtin_bit_cast(uint4, bv);
            }
          }
#pragma unroll
          for (int x = 0; x < TW; ++x)
#pragma unroll
            for (int y = 0; y < TW; ++y) O::mma(acc[x][y], A[x], B[y]);
        }
    }

    if (st != spb - 1) continue;
    // ---- block j complete
    const int nj = min(a.blk, a.L - j * a.blk);
    if constexpr (MODE == kStatsFull) {
      const int ct = j >> 6, kk = j & 63;
      uint8_t* kb_tile = a.kbp + ((size_t)bh * a.nct + ct) * G::SUB_BYTES;
      uint8_t* vb_tile = a.vbp + ((size_t)bh * a.nct + ct) * G::SUB_BYTES;
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int p = tid + 256 * u;
#pragma unroll
        for (int e = 0; e < KW; ++e) {  // add the four row quarters (adjacent lanes)
          csum[u][e] += __shfl_xor(csum[u][e], 1);
          csum[u][e] += __shfl_xor(csum[u][e], 2);
        }
        if (p < NTASK && (p & 3) == 0) {
          const int t = (p >> 2) / CG, g = (p >> 2) % CG;
#pragma unroll
          for (int e = 0; e < KW; ++e) {
            const int d = g * KW + e;
            const size_t o = ((size_t)bh * a.n + j) * D + d;
            if (t == 0) {
              a.qbar[o] = csum[u][e] / nj;
            } else if (t == 1) {
              const double kb = csum[u][e] / nj;
              a.kbar[o] = kb;
              kbf[d] = (float)kb;
              *(T*)(kb_tile + kfmt_offset<T, D>(kk, d)) = O::from_f32((float)kb);
            } else {
              a.vsum[o] = csum[u][e];
              vsf[d] = (float)csum[u][e];
              *(T*)(vb_tile + vfmt_offset<T, D>(kk, d)) = O::from_f32((float)csum[u][e]);
            }
          }
        }
#pragma unroll
        for (int e = 0; e < KW; ++e) csum[u][e] = 0.0;
      }
      __syncthreads();
      // Σ_n (k_n − k̄_j)ᵀ v_n = G_j − k̄_j ⊗ ΣV_j
#pragma unroll
      for (int x = 0; x < TW; ++x)
#pragma unroll
        for (int y = 0; y < TW; ++y)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            acc[x][y][r] -= kbf[32 * (dt0 + x) + vkey(r, h)] * vsf[32 * (et0 + y) + l32];
    } else if constexpr (MODE == kStatsMnorm) {
      double ss = 0.0;
#pragma unroll
      for (int x = 0; x < TW; ++x)
#pragma unroll
        for (int y = 0; y < TW; ++y)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int d = 32 * (dt0 + x) + vkey(r, h), e = 32 * (et0 + y) + l32;
            const double diff = (double)acc[x][y][r] - kbd[d] * vsd[e] - hb[x][y][r];
            ss += diff * diff;
            acc[x][y][r] = 0.0f;
          }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
      if (lane == 0) red[wv] = ss;
      __syncthreads();
      if (tid == 0) a.mnorm[bh * a.n + j] = sqrt(red[0] + red[1] + red[2] + red[3]);
    }
  }

  if constexpr (kDoPack) {
    __shared__ float kred[4];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) kn2max = fmaxf(kn2max, __shfl_xor(kn2max, o));
    if (lane == 0) kred[wv] = kn2max;
    __syncthreads();
    if (tid == 0)
      a.kmax2[(size_t)bh * a.nch + ch] = fmaxf(fmaxf(kred[0], kred[1]), fmaxf(kred[2], kred[3]));
  }
  if constexpr (MODE == kStatsFull) {
    float* dst = a.hpart + ((size_t)bh * a.nch + ch) * D * D;
#pragma unroll
    for (int x = 0; x < TW; ++x)
#pragma unroll
      for (int y = 0; y < TW; ++y)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int d = 32 * (dt0 + x) + vkey(r, h), e = 32 * (et0 + y) + l32;
          dst[d * D + e] = acc[x][y][r];
        }
  }
}

// H̄ = (1/n) Σ_runs (Σ_j H_j), summed in fp64; writes H̄ (fp64), its operand
// chunks for the fused kernel, and zeroes the padding rows of the k̄ / ΣV tiles.
template <typename T, int D>
__global__ __launch_bounds__(256) void k_hbar_reduce(StatsArgs a) {
  using G = Geo<T, D>;
  using O = Op<T>;
  constexpr int KW = G::KW, NC = G::NC;
  const long bh = blockIdx.x;
  const int x = blockIdx.y * 256 + threadIdx.x;
  if (x < D * D) {
    const int d = x / D, e = x % D;
    // the runs' partial sums in run order, loaded eight at a time so that the
    // loads are in flight together
    const float* hp = a.hpart + ((size_t)bh * a.nch * D + d) * D + e;
    double s = 0.0;
    int r = 0;
    for (; r + 8 <= a.nch; r += 8) {
      float x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = hp[(size_t)(r + u) * D * D];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += (double)x[u];
    }
    for (; r < a.nch; ++r) s += (double)hp[(size_t)r * D * D];
    const double hbv = s / a.n;
    a.hbar[(bh * D + d) * D + e] = hbv;
    const int et = e >> 5, lane = ((d % (2 * KW)) / KW) * 32 + (e & 31), c = d / (2 * KW), ee = d % KW;
    T* hbt = (T*)(a.hbt + (size_t)bh * D * D * G::ESZ);
    hbt[((et * NC + c) * kWave + lane) * KW + ee] = O::from_f32((float)hbv);
  }
  if (blockIdx.y == 0) {
    const int pad = a.nct * 64 - a.n;
    const int ct = a.nct - 1;
    uint8_t* kb_tile = a.kbp + ((size_t)bh * a.nct + ct) * G::SUB_BYTES;
    uint8_t* vb_tile = a.vbp + ((size_t)bh * a.nct + ct) * G::SUB_BYTES;
    for (int y = threadIdx.x; y < pad * D; y += 256) {
      const int kk = (a.n & 63) + y / D, d = y % D;
      *(T*)(kb_tile + kfmt_offset<T, D>(kk, d)) = O::from_f32(0.0f);
      *(T*)(vb_tile + vfmt_offset<T, D>(kk, d)) = O::from_f32(0.0f);
    }
  }
}

template <typename T, int D, bool SEG>
static hipError_t launch_stats_s(int mode, const StatsArgs& a, long bh, hipStream_t s) {
  dim3 grid((unsigned)(bh * a.nch));
  if (mode == kStatsFull)
    hipLaunchKernelGGL((k_block_stats<T, D, kStatsFull, SEG>), grid, dim3(256), 0, s, a);
  else if (mode == kStatsMnorm)
    hipLaunchKernelGGL((k_block_stats<T, D, kStatsMnorm, SEG>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((k_block_stats<T, D, kStatsPackOnly, SEG>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_stats_t(int mode, const StatsArgs& a, long bh, hipStream_t s) {
  return a.L0 < a.L ? launch_stats_s<T, D, true>(mode, a, bh, s)
                    : launch_stats_s<T, D, false>(mode, a, bh, s);
}

hipError_t launch_block_stats(int dtype, int D, int mode, const StatsArgs& a, long bh,
                              hipStream_t s) {
  if (dtype == 1) return D == 64 ? launch_stats_t<bf16, 64>(mode, a, bh, s)
                                 : launch_stats_t<bf16, 128>(mode, a, bh, s);
  return D == 64 ? launch_stats_t<float, 64>(mode, a, bh, s)
                 : launch_stats_t<float, 128>(mode, a, bh, s);
}

template <typename T, int D>
static hipError_t launch_reduce_t(const StatsArgs& a, long bh, hipStream_t s) {
  dim3 grid((unsigned)bh, (unsigned)((D * D + 255) / 256));
  hipLaunchKernelGGL((k_hbar_reduce<T, D>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_hbar_reduce(int dtype, int D, const StatsArgs& a, long bh, hipStream_t s) {
  if (dtype == 1) return D == 64 ? launch_reduce_t<bf16, 64>(a, bh, s)
                                 : launch_reduce_t<bf16, 128>(a, bh, s);
  return D == 64 ? launch_reduce_t<float, 64>(a, bh, s) : launch_reduce_t<float, 128>(a, bh, s);
}

}  // namespace pisa
