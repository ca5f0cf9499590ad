// Backward pass of PISA's zeroth-order-only variant (the authors' README,
// "Kernel variants": the _0th form is the one that supports training; the
// forward is the gist.science summary's "Core Algorithm" N_t equation without
// the first-order term). With the selection held fixed the forward is a
// softmax over an extended key set: the tokens of the selected blocks
// (weight 1, value v_n) and one centroid k̄_j per unselected block (weight
// n_j, value ΣV_j / n_j). For row t, p_tx = w_x e^{s q_t·K_x} / D_t and
// Δ_t = dO_t·o_t:
//   dS_tx = p̃_tx (dO_t·V'_x − w_x Δ_t),  p̃_tx = e^{s q_t·K_x} / D_t,
//   V'_x = v_n for a token, ΣV_j for a centroid (so w_x V_x = V'_x),
//   dq_t  = s Σ_x dS_tx K_x,
//   dk_n  = s Σ_t dS_tn q_t + (1/n_j) dk̄_j,  dk̄_j = s Σ_t dS_tj q_t,
//   dv_n  = Σ_t p̃_tn dO_t + dΣV_j,            dΣV_j = Σ_t p̃_tj dO_t,
// the token sums running over rows whose query block selects the block, the
// centroid sums over rows whose block leaves it out.
//
// Three kernels on one 64 x 64 tile engine. Each workgroup holds 64 query rows
// and 64 key entries in LDS (rows padded by 16 bytes); each of its four
// wavefronts forms one 32 x 32 quadrant of the logits and of dO·V' with
// v_mfma_f32_32x32x16_bf16 (f32: v_mfma_f32_32x32x2f32) over the head
// dimension, and takes the quadrant's weights straight from the accumulator
// registers as the A operand of the gradient product; the other operand is
// gathered from the LDS tile by the same key order (vkey, pisa_dev.h).
//   k_bwd_dq:  one workgroup per 64-row query tile: a first sweep over the
//              selected sub-tiles and the centroid tiles gives log2 D_t (an
//              online maximum), a second sweep dq; it stores log2 D_t and Δ_t.
//   k_bwd_dkv<centroid>: one workgroup per tile of 64 centroids, over every
//              query tile whose block leaves one of them out: dk̄, dΣV.
//   k_bwd_dkv<token>: one workgroup per 64-key sub-tile, over the query
//              blocks that select its block (a bitmap of the selection):
//              dk, dv, plus dk̄_j / n_j and dΣV_j.
// Every sum runs in a fixed order: the results are deterministic.
#include "pisa_dev.h"
#include "pisa_internal.h"

namespace pisa {

namespace {

constexpr float kInf = __builtin_huge_valf();

template <typename T, int D>
struct BT {
  using G = Geo<T, D>;
  static constexpr int KW = G::KW, ESZ = G::ESZ, NC = G::NC, DT = G::DT, CPK = G::CPK;
  static constexpr int CPR = G::CPR;             // 16-byte chunks per row
  static constexpr int RP = D * ESZ + 16;        // LDS row pitch in bytes
  static constexpr int TILE = 64 * RP;           // one 64-row tile in LDS
  static constexpr int PER = 64 * CPR / 256;     // chunks per thread to stage a tile
  static constexpr int XF = 2 * DT * 16 * 64;    // floats of one partial-sum exchange
};

// Operand for a contraction over d: rows of the 32-row half rh of a tile.
template <typename T, int D>
__device__ __forceinline__ uint4 op_row(const uint8_t* tile, int rh, int c, int lane) {
  using B = BT<T, D>;
  const int row = 32 * rh + (lane & 31);
  const int d0 = 2 * B::KW * c + B::KW * (lane >> 5);
  return *(const uint4*)(tile + row * B::RP + d0 * B::ESZ);
}

// B operand for a contraction over the rows of the 32-row half rh (in vkey
// order, matching an accumulator used as the A operand), column d = 32 dt + l%32.
template <typename T, int D>
__device__ __forceinline__ uint4 op_col(const uint8_t* tile, int rh, int dt, int c, int lane) {
  using B = BT<T, D>;
  const int d = 32 * dt + (lane & 31), h = lane >> 5;
  T vals[B::KW];
#pragma unroll
  for (int e = 0; e < B::KW; ++e)
    vals[e] = *(const T*)(tile + (32 * rh + vkey(B::KW * c + e, h)) * B::RP + d * B::ESZ);
  return __builtin_bit_cast(uint4, vals);
}

// Byte offset of token row `row` of head bh in a q, k, v, o or gradient tensor.
__device__ __forceinline__ size_t row_off(const BwdArgs& a, long bh, int row) {
  return (size_t)(bh / a.H) * a.stride_b + (size_t)(bh % a.H) * a.stride_h + (size_t)row * a.stride_l;
}

// Rows r0 .. r0+63 of a tensor into an LDS tile (zero past L).
template <typename T, int D>
__device__ __forceinline__ void stage_rows(uint8_t* tile, const uint8_t* src, const BwdArgs& a, long bh,
                                           int r0) {
  using B = BT<T, D>;
#pragma unroll
  for (int i = 0; i < B::PER; ++i) {
    const int x = threadIdx.x + 256 * i, row = x / B::CPR, cc = x % B::CPR;
    const int g = r0 + row;
    const uint4 val = g < a.L ? *(const uint4*)(src + row_off(a, bh, g) + cc * 16) : make_uint4(0, 0, 0, 0);
    *(uint4*)(tile + row * B::RP + cc * 16) = val;
  }
}

// Rows 64 ct .. 64 ct + 63 of an fp64 [n][D] statistic of head bh, rounded to T
// (zero past n).
template <typename T, int D>
__device__ __forceinline__ void stage_stat(uint8_t* tile, const double* src, const BwdArgs& a, long bh,
                                           int ct) {
  using B = BT<T, D>;
  using O = Op<T>;
#pragma unroll
  for (int i = 0; i < B::PER; ++i) {
    const int x = threadIdx.x + 256 * i, row = x / B::CPR, cc = x % B::CPR;
    const int j = 64 * ct + row;
    T vals[B::KW];
#pragma unroll
    for (int e = 0; e < B::KW; ++e)
      vals[e] = O::from_f32(j < a.n ? (float)src[((size_t)bh * a.n + j) * D + cc * B::KW + e] : 0.0f);
    *(uint4*)(tile + row * B::RP + cc * 16) = __builtin_bit_cast(uint4, vals);
  }
}

// Is key block j selected by query block i (head bh)?
__device__ __forceinline__ bool selected(const BwdArgs& a, long bh, int i, int j) {
  return (a.selmap[((size_t)bh * a.n + i) * a.W + (j >> 5)] >> (j & 31)) & 1u;
}

// Bits of centroids 64 ct .. 64 ct + 63 selected by query block i.
__device__ __forceinline__ unsigned long long selected64(const BwdArgs& a, long bh, int i, int ct) {
  const uint32_t* row = a.selmap + ((size_t)bh * a.n + i) * a.W;
  const unsigned long long lo = row[2 * ct];
  const unsigned long long hi = 2 * ct + 1 < a.W ? row[2 * ct + 1] : 0u;
  return lo | (hi << 32);
}

// Sums the partial accumulators of the two wavefronts that share output rows
// (wavefront `part` 1 hands its half to `part` 0 through LDS); afterwards the
// `part` 0 wavefronts hold the totals.
template <int DT>
__device__ __forceinline__ void merge_halves(f32x16 (&acc)[DT], float* xf, int slot, int part, int lane) {
  if (part == 1)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) xf[((slot * DT + dt) * 16 + r) * 64 + lane] = acc[dt][r];
  __syncthreads();
  if (part == 0)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[dt][r] += xf[((slot * DT + dt) * 16 + r) * 64 + lane];
}

// ---------------------------------------------------------------------------
// dq, with the rows' log2 D_t and Δ_t. Wavefront w = (xh, th): Sᵀ quadrant of
// key half xh x row half th; its dq partial covers rows th and sums keys xh.
template <typename T, int D, int SPB>
__global__ __launch_bounds__(256, 1) void k_bwd_dq(BwdArgs a) {
  using B = BT<T, D>;
  constexpr int KW = B::KW, NC = B::NC, DT = B::DT, CPK = B::CPK;
  __shared__ __align__(16) uint8_t qt[B::TILE], ot[B::TILE];
  __shared__ __align__(16) uint8_t kv[2 * B::TILE];  // key and value tiles; partial sums at the end
  __shared__ float lse_s[64], dl_s[64], wx_s[64];
  __shared__ float stat[2][2][2][32];  // [key half][row half][max, sum][row]
  __shared__ uint32_t selw[kMaxBlocks / 32];
  uint8_t* kt = kv;
  uint8_t* vt = kv + B::TILE;

  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int w = tid >> 6, th = w & 1, xh = w >> 1;
  const long item = blockIdx.x;
  const int half = (int)(item % SPB);
  const long rest = item / SPB;
  const int i = (int)(rest % a.n);
  const long bh = rest / a.n;
  const int r0 = i * a.blk + half * 64;
  if (r0 >= a.L) return;
  const float cs = a.scale * kLog2e;

  stage_rows<T, D>(qt, a.q, a, bh, r0);
  stage_rows<T, D>(ot, a.dout, a, bh, r0);
  for (int x = tid; x < a.W; x += 256) selw[x] = a.selmap[((size_t)bh * a.n + i) * a.W + x];
  {  // Δ_t = dO_t·o_t, four threads per row
    const int row = tid >> 2, part = tid & 3, g = r0 + row;
    float acc = 0.0f;
    if (g < a.L) {
      const uint8_t* po = a.o + row_off(a, bh, g);
      const uint8_t* pd = a.dout + row_off(a, bh, g);
      for (int cc = part; cc < B::CPR; cc += 4) {
        float xo[KW], xd[KW];
        Op<T>::unpack(*(const uint4*)(po + cc * 16), xo);
        Op<T>::unpack(*(const uint4*)(pd + cc * 16), xd);
#pragma unroll
        for (int e = 0; e < KW; ++e) acc = fmaf(xo[e], xd[e], acc);
      }
    }
    acc += __shfl_xor(acc, 1);
    acc += __shfl_xor(acc, 2);
    if (part == 0) dl_s[row] = acc;
  }
  __syncthreads();

  // the key tiles of this query tile: the selected blocks' 64-key sub-tiles,
  // then the centroid tiles
  const int nsub = a.topk * SPB;
  const int ntile = nsub + a.nct;
  const int32_t* myidx = a.idx + ((size_t)bh * a.n + i) * a.topk;
  // stages tile u; returns false for a sub-tile past the end of the sequence
  auto stage = [&](int u, bool values) -> bool {
    if (u < nsub) {
      const int j = min(max(myidx[u / SPB], 0), a.n - 1), st = u % SPB;
      const int k0 = j * a.blk + st * 64;
      if (k0 >= a.L) return false;
      stage_rows<T, D>(kt, a.k, a, bh, k0);
      if (values) stage_rows<T, D>(vt, a.v, a, bh, k0);
      if (tid < 64) wx_s[tid] = k0 + tid < a.L ? 1.0f : -1.0f;
    } else {
      const int ct = u - nsub;
      stage_stat<T, D>(kt, a.kbar, a, bh, ct);
      if (values) stage_stat<T, D>(vt, a.vsum, a, bh, ct);
      if (tid < 64) {
        const int j = 64 * ct + tid;
        const bool sel = j < a.n && ((selw[j >> 5] >> (j & 31)) & 1u);
        wx_s[tid] = (j < a.n && !sel) ? (float)(j == a.n - 1 ? a.n_last : a.blk) : -1.0f;
      }
    }
    return true;
  };

  // ---- sweep 1: log2 D_t with an online maximum (per lane: column t)
  float m = -kInf, l = 0.0f;
  for (int u = 0; u < ntile; ++u) {
    __syncthreads();  // tiles free
    const bool live = stage(u, false);
    __syncthreads();
    if (!live) continue;
    f32x16 sacc = f32x16{};
#pragma unroll
    for (int c = 0; c < NC; ++c) Op<T>::mma(sacc, op_row<T, D>(kt, xh, c, lane), op_row<T, D>(qt, th, c, lane));
    float tmax = -kInf;
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (wx_s[32 * xh + vkey(r, h)] >= 0.0f) tmax = fmaxf(tmax, sacc[r] * cs);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    if (tmax == -kInf) continue;
    const float mn = fmaxf(m, tmax);
    float sum = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float wx = wx_s[32 * xh + vkey(r, h)];
      if (wx >= 0.0f) sum += wx * __builtin_amdgcn_exp2f(sacc[r] * cs - mn);
    }
    sum += __shfl_xor(sum, 32);
    l = l * __builtin_amdgcn_exp2f(m - mn) + sum;
    m = mn;
  }
  // combine the two key halves of each row
  if (h == 0) {
    stat[xh][th][0][l32] = m;
    stat[xh][th][1][l32] = l;
  }
  __syncthreads();
  if (xh == 0 && h == 0) {
    const float m1 = stat[1][th][0][l32], l1 = stat[1][th][1][l32];
    const float mm = fmaxf(m, m1);
    const float ll = l * __builtin_amdgcn_exp2f(m - mm) + l1 * __builtin_amdgcn_exp2f(m1 - mm);
    const int t = 32 * th + l32, g = r0 + t;
    const float v2 = g < a.L ? mm + __log2f(ll) : kInf;  // padding rows: every weight 0
    lse_s[t] = v2;
    if (g < a.L) {
      a.lse[(size_t)bh * a.n * a.blk + g] = v2;
      a.delta[(size_t)bh * a.n * a.blk + g] = dl_s[t];
    }
  }

  // ---- sweep 2: dq_t = s Σ_x dS_tx K_x
  f32x16 dq[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dq[dt] = f32x16{};
  for (int u = 0; u < ntile; ++u) {
    __syncthreads();
    const bool live = stage(u, true);
    __syncthreads();
    if (!live) continue;
    f32x16 sacc = f32x16{}, pacc = f32x16{};
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      Op<T>::mma(sacc, op_row<T, D>(kt, xh, c, lane), op_row<T, D>(qt, th, c, lane));
      Op<T>::mma(pacc, op_row<T, D>(vt, xh, c, lane), op_row<T, D>(ot, th, c, lane));
    }
    const int t = 32 * th + l32;
    const float lt = lse_s[t], dlt = dl_s[t];
    float ds[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float wx = wx_s[32 * xh + vkey(r, h)];
      const float p = wx >= 0.0f ? __builtin_amdgcn_exp2f(sacc[r] * cs - lt) : 0.0f;
      ds[r] = p * (pacc[r] - fmaxf(wx, 0.0f) * dlt);
    }
#pragma unroll
    for (int c = 0; c < CPK; ++c) {
      const uint4 av = Op<T>::pack(&ds[KW * c]);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) Op<T>::mma(dq[dt], av, op_col<T, D>(kt, xh, dt, c, lane));
    }
  }
  __syncthreads();
  merge_halves<DT>(dq, (float*)kv, th, xh, lane);
  if (xh == 0) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int g = r0 + 32 * th + vkey(r, h);
        if (g < a.L)
          *(T*)(a.dq + row_off(a, bh, g) + (32 * dt + l32) * B::ESZ) = Op<T>::from_f32(a.scale * dq[dt][r]);
      }
  }
}

// ---------------------------------------------------------------------------
// dk and dv of one 64-entry key tile: wavefront w = (th, xh) forms the S
// quadrant of row half th x key half xh; its dk / dv partial covers keys xh
// and sums rows th. CENT: a tile of 64 centroids, gradients of k̄ and ΣV (fp32,
// to the workspace); otherwise a 64-key sub-tile of block j, whose final dk,
// dv take the centroid gradients of j too.
template <typename T, int D, int SPB, bool CENT>
__global__ __launch_bounds__(256, 1) void k_bwd_dkv(BwdArgs a) {
  using B = BT<T, D>;
  constexpr int KW = B::KW, NC = B::NC, DT = B::DT, CPK = B::CPK;
  __shared__ __align__(16) uint8_t tiles[4 * B::TILE];  // k, v, q, dO; partial sums at the end
  __shared__ float lse_s[64], dl_s[64], wx_s[64];
  uint8_t* kt = tiles;
  uint8_t* vt = tiles + B::TILE;
  uint8_t* qt = tiles + 2 * B::TILE;
  uint8_t* ot = tiles + 3 * B::TILE;
  static_assert(4 * B::TILE >= 2 * B::XF * 4, "exchange fits in the tiles");

  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int w = tid >> 6, xh = w & 1, th = w >> 1;
  const float cs = a.scale * kLog2e;
  long bh;
  int j = 0, ct = 0, k0 = 0;
  if constexpr (CENT) {
    bh = blockIdx.x / a.nct;
    ct = (int)(blockIdx.x % a.nct);
  } else {
    const int st = (int)(blockIdx.x % SPB);
    const long rest = blockIdx.x / SPB;
    j = (int)(rest % a.n);
    bh = rest / a.n;
    k0 = j * a.blk + st * 64;
    if (k0 >= a.L) return;
  }

  if constexpr (CENT) {
    stage_stat<T, D>(kt, a.kbar, a, bh, ct);
    stage_stat<T, D>(vt, a.vsum, a, bh, ct);
    if (tid < 64) {
      const int jc = 64 * ct + tid;
      wx_s[tid] = jc < a.n ? (float)(jc == a.n - 1 ? a.n_last : a.blk) : -1.0f;
    }
  } else {
    stage_rows<T, D>(kt, a.k, a, bh, k0);
    stage_rows<T, D>(vt, a.v, a, bh, k0);
    if (tid < 64) wx_s[tid] = k0 + tid < a.L ? 1.0f : -1.0f;
  }
  // centroids that exist in this tile (bit x: centroid 64 ct + x)
  const int nvalid_c = CENT ? min(64, a.n - 64 * ct) : 64;
  const unsigned long long valid_c = nvalid_c >= 64 ? ~0ull : ((1ull << nvalid_c) - 1ull);

  f32x16 dk[DT], dv[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dk[dt] = dv[dt] = f32x16{};

  // one 64-row query tile against the key tile; cmask: centroids the query
  // block selects (they take no weight from its rows)
  auto query_tile = [&](int r0, unsigned long long cmask) {
    __syncthreads();  // q / dO tiles free
    stage_rows<T, D>(qt, a.q, a, bh, r0);
    stage_rows<T, D>(ot, a.dout, a, bh, r0);
    if (tid < 64) {
      const int g = r0 + tid;
      lse_s[tid] = g < a.L ? a.lse[(size_t)bh * a.n * a.blk + g] : kInf;
      dl_s[tid] = g < a.L ? a.delta[(size_t)bh * a.n * a.blk + g] : 0.0f;
    }
    __syncthreads();
    f32x16 sacc = f32x16{}, pacc = f32x16{};
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      Op<T>::mma(sacc, op_row<T, D>(qt, th, c, lane), op_row<T, D>(kt, xh, c, lane));
      Op<T>::mma(pacc, op_row<T, D>(ot, th, c, lane), op_row<T, D>(vt, xh, c, lane));
    }
    const int x = 32 * xh + l32;
    const float wx = wx_s[x];
    const bool live = wx >= 0.0f && !((cmask >> x) & 1ull);
    float p[16], ds[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = 32 * th + vkey(r, h);
      p[r] = live ? __builtin_amdgcn_exp2f(sacc[r] * cs - lse_s[t]) : 0.0f;
      ds[r] = p[r] * (pacc[r] - wx * dl_s[t]);
    }
#pragma unroll
    for (int c = 0; c < CPK; ++c) {
      const uint4 pv = Op<T>::pack(&p[KW * c]);
      const uint4 dsv = Op<T>::pack(&ds[KW * c]);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        Op<T>::mma(dv[dt], pv, op_col<T, D>(ot, th, dt, c, lane));
        Op<T>::mma(dk[dt], dsv, op_col<T, D>(qt, th, dt, c, lane));
      }
    }
  };

  if constexpr (CENT) {
    for (int i = 0; i < a.n; ++i) {
      const unsigned long long cm = selected64(a, bh, i, ct);
      if ((cm & valid_c) == valid_c) continue;  // the block selects every centroid here
      for (int hf = 0; hf < SPB; ++hf) {
        const int r0 = i * a.blk + hf * 64;
        if (r0 < a.L) query_tile(r0, cm);
      }
    }
  } else {
    // the query blocks that select block j, ascending, 64 at a time
    for (int ib = 0; ib < a.n; ib += 64) {
      const int i = ib + lane;
      unsigned long long bits = __ballot(i < a.n && selected(a, bh, i, j));
      while (bits) {
        const int ii = ib + __ffsll(bits) - 1;
        bits &= bits - 1ull;
        for (int hf = 0; hf < SPB; ++hf) {
          const int r0 = ii * a.blk + hf * 64;
          if (r0 < a.L) query_tile(r0, 0ull);
        }
      }
    }
  }

  __syncthreads();  // tiles free: partial sums of the two row halves meet there
  float* xf = (float*)tiles;
  merge_halves<DT>(dk, xf, xh, th, lane);
  merge_halves<DT>(dv, xf + 2 * DT * 16 * 64, xh, th, lane);
  if (th != 0) return;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int x = 32 * xh + vkey(r, h), d = 32 * dt + l32;
      if constexpr (CENT) {
        const int jc = 64 * ct + x;
        if (jc < a.n) {
          a.dkbar[((size_t)bh * a.n + jc) * D + d] = a.scale * dk[dt][r];
          a.dvsum[((size_t)bh * a.n + jc) * D + d] = dv[dt][r];
        }
      } else {
        const int g = k0 + x;
        if (g < a.L) {
          const float nj = (float)(j == a.n - 1 ? a.n_last : a.blk);
          const size_t sidx = ((size_t)bh * a.n + j) * D + d;
          const float gk = a.scale * dk[dt][r] + a.dkbar[sidx] / nj;
          const float gv = dv[dt][r] + a.dvsum[sidx];
          *(T*)(a.dk + row_off(a, bh, g) + d * B::ESZ) = Op<T>::from_f32(gk);
          *(T*)(a.dv + row_off(a, bh, g) + d * B::ESZ) = Op<T>::from_f32(gv);
        }
      }
    }
}

// Selection bitmap: zeroed, then bit j of row i set for each selected block.
__global__ void k_bwd_selmap_clear(uint32_t* m, size_t words) {
  for (size_t x = (size_t)blockIdx.x * 256 + threadIdx.x; x < words; x += (size_t)gridDim.x * 256) m[x] = 0u;
}

__global__ void k_bwd_selmap_set(BwdArgs a) {
  const long row = blockIdx.x;  // (bh, i)
  const int32_t* ix = a.idx + row * a.topk;
  uint32_t* m = a.selmap + row * a.W;
  for (int s = threadIdx.x; s < a.topk; s += 256) {
    const int j = min(max(ix[s], 0), a.n - 1);
    atomicOr(&m[j >> 5], 1u << (j & 31));
  }
}

template <typename T, int D, int SPB>
hipError_t launch_bwd_t(const BwdArgs& a, long bh, hipStream_t s) {
  const size_t words = (size_t)bh * a.n * a.W;
  hipLaunchKernelGGL(k_bwd_selmap_clear, dim3(1024), dim3(256), 0, s, a.selmap, words);
  hipLaunchKernelGGL(k_bwd_selmap_set, dim3((unsigned)(bh * a.n)), dim3(256), 0, s, a);
  hipLaunchKernelGGL((k_bwd_dq<T, D, SPB>), dim3((unsigned)(bh * a.n * SPB)), dim3(256), 0, s, a);
  hipLaunchKernelGGL((k_bwd_dkv<T, D, SPB, true>), dim3((unsigned)(bh * a.nct)), dim3(256), 0, s, a);
  hipLaunchKernelGGL((k_bwd_dkv<T, D, SPB, false>), dim3((unsigned)(bh * a.n * SPB)), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_bwd_b(const BwdArgs& a, long bh, hipStream_t s) {
  return a.blk == 64 ? launch_bwd_t<T, D, 1>(a, bh, s) : launch_bwd_t<T, D, 2>(a, bh, s);
}

}  // namespace

hipError_t launch_bwd(int dtype, int D, const BwdArgs& a, long bh, hipStream_t s) {
  if (dtype == 1) return D == 64 ? launch_bwd_b<bf16, 64>(a, bh, s) : launch_bwd_b<bf16, 128>(a, bh, s);
  return D == 64 ? launch_bwd_b<float, 64>(a, bh, s) : launch_bwd_b<float, 128>(a, bh, s);
}

}  // namespace pisa
