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
//              online maximum; skipped when the forward pass handed over
//              ln D_t), a second sweep dq; it stores log2 D_t and Δ_t.
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
// Query blocks listed at a time by a key tile's workgroup: the list's LDS
// stays small enough for two bf16 workgroups of k_bwd_dkv per compute unit.
constexpr int kQChunk = 4096;

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
// For 16-bit elements the eight rows of a lane are rows r0..r0+3 and
// r0+8..r0+11 (r0 = 32 rh + 16 c + 4 h), read with two transposing LDS loads:
// in each group of 16 lanes, lane j points at 4 elements of row r0 + j/4
// starting at column 32 dt + 16 (group & 1) + 4 (j % 4), and every lane of the
// group receives its own column from the four rows.
typedef short bwd_v4s __attribute__((ext_vector_type(4)));
template <typename T, int D>
__device__ __forceinline__ uint4 op_col(const uint8_t* tile, int rh, int dt, int c, int lane) {
  using B = BT<T, D>;
  const int h = lane >> 5;
  if constexpr (B::ESZ == 2) {
    const int g = lane >> 4, j = lane & 15;
    const int row = 32 * rh + 16 * c + 4 * h + (j >> 2);
    const int col = 32 * dt + 16 * (g & 1) + 4 * (j & 3);
    const uint8_t* p = tile + row * B::RP + col * 2;
    typedef __attribute__((address_space(3))) bwd_v4s* lds_v4s;
    const bwd_v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)p);
    const bwd_v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(p + 8 * B::RP));
    const uint2 a = __builtin_bit_cast(uint2, lo), b = __builtin_bit_cast(uint2, hi);
    return make_uint4(a.x, a.y, b.x, b.y);
  } else {
    const int d = 32 * dt + (lane & 31);
    T vals[B::KW];
#pragma unroll
    for (int e = 0; e < B::KW; ++e)
      vals[e] = *(const T*)(tile + (32 * rh + vkey(B::KW * c + e, h)) * B::RP + d * B::ESZ);
    return __builtin_bit_cast(uint4, vals);
  }
}

// Byte offset of token row `row` of head bh in a q, k, v, o or gradient tensor.
__device__ __forceinline__ size_t row_off(const BwdArgs& a, long bh, int row) {
  return (size_t)(bh / a.H) * a.stride_b + (size_t)(bh % a.H) * a.stride_h + (size_t)row * a.stride_l;
}

// A run of rows: row g at base + g * pitch, rows from `limit` on read as zero.
struct Rows {
  const uint8_t* base;
  size_t pitch;
  int limit;
};

__device__ __forceinline__ Rows tensor_rows(const BwdArgs& a, const uint8_t* t, long bh) {
  return Rows{t + row_off(a, bh, 0), a.stride_l, a.L};
}

template <typename T, int D>
__device__ __forceinline__ Rows centroid_rows(const BwdArgs& a, const uint8_t* t, long bh) {
  return Rows{t + (size_t)bh * a.nct * 64 * D * sizeof(T), (size_t)D * sizeof(T), a.nct * 64};
}

// Issues the loads of rows r0 .. r0+63 into registers (one tile's share of this thread).
template <typename T, int D>
__device__ __forceinline__ void load_rows(const Rows& s, int r0, uint4 (&pre)[BT<T, D>::PER]) {
  using B = BT<T, D>;
#pragma unroll
  for (int i = 0; i < B::PER; ++i) {
    const int x = threadIdx.x + 256 * i, row = x / B::CPR, cc = x % B::CPR;
    const int g = r0 + row;
    pre[i] = g < s.limit ? *(const uint4*)(s.base + (size_t)g * s.pitch + cc * 16) : make_uint4(0, 0, 0, 0);
  }
}

template <typename T, int D>
__device__ __forceinline__ void store_rows(uint8_t* tile, const uint4 (&pre)[BT<T, D>::PER]) {
  using B = BT<T, D>;
#pragma unroll
  for (int i = 0; i < B::PER; ++i) {
    const int x = threadIdx.x + 256 * i, row = x / B::CPR, cc = x % B::CPR;
    *(uint4*)(tile + row * B::RP + cc * 16) = pre[i];
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
// Both sweeps run over the same key tiles (the selected blocks' 64-key
// sub-tiles, then the centroid tiles); the rows of tile u+1 load into
// registers while tile u is computed.
// The tile of workgroup wg in the XCD-aware order of the forward pass:
// workgroups reach the chip's eight XCDs in turn, and within every full
// generation of nwg workgroups those of one XCD take consecutive tiles of one
// head, so the blocks they gather meet in that XCD's L2. A last, partial
// generation keeps the plain order.
__device__ __forceinline__ long bwd_tile_of(long wg, long nwg, long total) {
  const long g = wg / nwg;
  if ((g + 1) * nwg > total || (nwg & 7) != 0) return wg;
  const long r = wg - g * nwg;
  return g * nwg + (r & 7) * (nwg >> 3) + (r >> 3);
}

// k_bwd_dq runs in generations of as many workgroups as are resident, like the
// forward pass: before its sweep a workgroup of generation g waits until every
// workgroup of generation g-1 is past its selected sub-tiles, so the resident
// ascending sweeps over the gathered blocks stay in step and one XCD's L2
// serves each block to many of them. Every query tile has the same work (topk
// blocks, then the centroid tiles). The wait is bounded by sync_ticks and
// decides no result.
template <typename T, int D, int SPB>
__global__ __launch_bounds__(256, 1) void k_bwd_dq(BwdArgs a) {
  using B = BT<T, D>;
  constexpr int KW = B::KW, NC = B::NC, DT = B::DT, CPK = B::CPK, PER = B::PER;
  __shared__ __align__(16) uint8_t qt[B::TILE], ot[B::TILE];
  __shared__ __align__(16) uint8_t kv[2 * B::TILE];  // key and value tiles; partial sums at the end
  __shared__ float lse_s[64], dl_s[64], wx_s[64];
  __shared__ float stat[2][2][2][32];  // [key half][row half][max, sum][row]
  __shared__ uint32_t selw[kMaxBlocks / 32];
  uint8_t* kt = kv;
  uint8_t* vt = kv + B::TILE;

  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int w = tid >> 6, th = w & 1, xh = w >> 1;
  const long g = (long)blockIdx.x / a.nwg_dq;
  const long item = bwd_tile_of(blockIdx.x, a.nwg_dq, a.total);
  auto done = [&]() {
    if (tid == 0) __hip_atomic_fetch_add(a.sync, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  const int half = (int)(item % SPB);
  const long rest = item / SPB;
  const int i = (int)(rest % a.n);
  const long bh = rest / a.n;
  const int r0 = i * a.blk + half * 64;
  if (r0 >= a.L) {
    done();
    return;
  }
  const float cs = a.scale * kLog2e;

  const Rows krows = tensor_rows(a, a.k, bh), vrows = tensor_rows(a, a.v, bh);
  const Rows kbrows = centroid_rows<T, D>(a, a.kbt, bh), vbrows = centroid_rows<T, D>(a, a.vbt, bh);
  const int nsub = a.topk * SPB;
  const int ntile = nsub + a.nct;
  const int32_t* myidx = a.idx + ((size_t)bh * a.n + i) * a.topk;
  // first row of key tile u in its source (a sub-tile past the sequence reads as zeros)
  auto tile_r0 = [&](int u) {
    if (u < nsub) return min(max(myidx[u / SPB], 0), a.n - 1) * a.blk + (u % SPB) * 64;
    return 64 * (u - nsub);
  };
  uint4 pk[PER], pv[PER];
  auto prefetch_into = [&](int u, bool values, uint4 (&xk)[PER], uint4 (&xv)[PER]) {
    const int k0 = tile_r0(u);
    load_rows<T, D>(u < nsub ? krows : kbrows, k0, xk);
    if (values) load_rows<T, D>(u < nsub ? vrows : vbrows, k0, xv);
  };
  auto prefetch = [&](int u, bool values) { prefetch_into(u, values, pk, pv); };
  // weight of each key of tile u: 1 for a token, n_j for an unselected
  // centroid, -1 for no key (past the sequence, padding, selected centroid)
  auto set_weights = [&](int u) {
    if (tid >= 64) return;
    if (u < nsub) {
      wx_s[tid] = tile_r0(u) + tid < a.L ? 1.0f : -1.0f;
    } else {
      const int j = 64 * (u - nsub) + tid;
      const bool sel = j < a.n && ((selw[j >> 5] >> (j & 31)) & 1u);
      wx_s[tid] = (j < a.n && !sel) ? (float)(j == a.n - 1 ? a.n_last : a.blk) : -1.0f;
    }
  };

  // ln D_t from the forward pass makes the first sweep unnecessary
  const bool have_lse = a.lse_in != nullptr;
  {
    uint4 pq[PER], po[PER];
    load_rows<T, D>(tensor_rows(a, a.q, bh), r0, pq);
    load_rows<T, D>(tensor_rows(a, a.dout, bh), r0, po);
    store_rows<T, D>(qt, pq);
    store_rows<T, D>(ot, po);
  }
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
  if (g > 0) {  // the generation wait
    if (tid == 0) {
      const int target = (int)(g * a.nwg_dq);
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      while (__hip_atomic_load(a.sync, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target &&
             __builtin_amdgcn_s_memrealtime() - t0 < (uint64_t)a.sync_ticks)
        __builtin_amdgcn_s_sleep(2);
    }
    __syncthreads();
  }
  prefetch(0, have_lse);

  // ---- sweep 1: log2 D_t with an online maximum (per lane: column t)
  float m = -kInf, l = 0.0f;
  for (int u = 0; u < (have_lse ? 0 : ntile); ++u) {
    __syncthreads();  // tiles free
    store_rows<T, D>(kt, pk);
    set_weights(u);
    __syncthreads();
    if (u + 1 < ntile) prefetch(u + 1, false);
    else prefetch(0, true);  // the first tile of the second sweep
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
    float v2 = kInf;  // padding rows: every weight 0
    if (g < a.L) v2 = have_lse ? a.lse_in[(size_t)bh * a.L + g] * kLog2e : mm + __log2f(ll);
    lse_s[t] = v2;
    if (g < a.L) {
      a.lse[(size_t)bh * a.n * a.blk + g] = v2;
      a.delta[(size_t)bh * a.n * a.blk + g] = dl_s[t];
    }
  }

  // ---- sweep 2: dq_t = s Σ_x dS_tx K_x. The rows of two tiles are in flight
  // in registers (tiles u+1 and u+2 load while tile u is computed), so a
  // gathered block that misses the L2 has two tiles' compute to arrive. Built
  // with every MFMA result in VGPRs this takes 237 registers per lane (bf16,
  // D = 128), two wavefronts per SIMD; built with the accumulators in AGPRs it
  // takes 292, one wavefront per SIMD, and the backward ran 90.0 -> 110.7 ms
  // at the Wan shape instead of 90.0 -> 87.2 ms.
  f32x16 dq[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dq[dt] = f32x16{};
  uint4 pk2[PER], pv2[PER];
  if (ntile > 1) prefetch_into(1, true, pk2, pv2);
  auto tile = [&](int u, uint4 (&xk)[PER], uint4 (&xv)[PER]) {
    if (u == nsub) done();  // past the selected sub-tiles: the centroid tiles follow
    __syncthreads();
    store_rows<T, D>(kt, xk);
    store_rows<T, D>(vt, xv);
    set_weights(u);
    __syncthreads();
    if (u + 2 < ntile) prefetch_into(u + 2, true, xk, xv);
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
  };
  for (int u = 0; u < ntile; u += 2) {
    tile(u, pk, pv);
    if (u + 1 < ntile) tile(u + 1, pk2, pv2);
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
// dv take the centroid gradients of j too. The query blocks visited (those
// that select block j; for centroids, those that leave one of the tile's
// centroids out) are listed first, ascending, so the rows of the next query
// tile load into registers while the current one is computed.
template <typename T, int D, int SPB, bool CENT>
__global__ __launch_bounds__(256, 2) void k_bwd_dkv(BwdArgs a) {
  using B = BT<T, D>;
  constexpr int KW = B::KW, NC = B::NC, DT = B::DT, CPK = B::CPK, PER = B::PER;
  __shared__ __align__(16) uint8_t tiles[4 * B::TILE];  // k, v, q, dO; partial sums at the end
  __shared__ float lse_s[64], dl_s[64], wx_s[64];
  __shared__ uint16_t qlist[kQChunk];
  __shared__ int qcount, qnext;
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
  int i_lo = 0, i_hi = a.n, part = 0;  // the query blocks this workgroup visits lie in [i_lo, i_hi)
  if constexpr (CENT) {
    part = (int)(blockIdx.x % a.cparts);
    const long rest = blockIdx.x / a.cparts;
    bh = rest / a.nct;
    ct = (int)(rest % a.nct);
    i_lo = (int)((long)part * a.n / a.cparts);
    i_hi = (int)((long)(part + 1) * a.n / a.cparts);
  } else {
    const long item = bwd_tile_of(blockIdx.x, a.nwg_dkv, a.total);
    const int st = (int)(item % SPB);
    const long rest = item / SPB;
    j = (int)(rest % a.n);
    bh = rest / a.n;
    k0 = j * a.blk + st * 64;
    if (k0 >= a.L) return;
  }
  // centroids that exist in this tile (bit x: centroid 64 ct + x)
  const int nvalid_c = CENT ? min(64, a.n - 64 * ct) : 64;
  const unsigned long long valid_c = nvalid_c >= 64 ? ~0ull : ((1ull << nvalid_c) - 1ull);

  // the query blocks to visit, ascending, listed by wavefront 0 in chunks of
  // at most kQChunk, the scan of query blocks resuming at `from`
  auto list_chunk = [&](int from) {
    if (w != 0) return;
    int cnt = 0, ib = from;
    for (; ib < i_hi && cnt <= kQChunk - 64; ib += 64) {
      const int i = ib + lane;
      bool take = false;
      if (i < i_hi) {
        if constexpr (CENT) take = (selected64(a, bh, i, ct) & valid_c) != valid_c;
        else take = selected(a, bh, i, j);
      }
      const unsigned long long bits = __ballot(take);
      if (take) qlist[cnt + __popcll(bits & ((1ull << lane) - 1ull))] = (uint16_t)i;
      cnt += __popcll(bits);
    }
    if (lane == 0) {
      qcount = cnt;
      qnext = ib;
    }
  };
  list_chunk(i_lo);
  {
    uint4 pk[PER], pv[PER];
    const Rows kr = CENT ? centroid_rows<T, D>(a, a.kbt, bh) : tensor_rows(a, a.k, bh);
    const Rows vr = CENT ? centroid_rows<T, D>(a, a.vbt, bh) : tensor_rows(a, a.v, bh);
    const int kr0 = CENT ? 64 * ct : k0;
    load_rows<T, D>(kr, kr0, pk);
    load_rows<T, D>(vr, kr0, pv);
    store_rows<T, D>(kt, pk);
    store_rows<T, D>(vt, pv);
  }
  if (tid < 64) {
    if constexpr (CENT) {
      const int jc = 64 * ct + tid;
      wx_s[tid] = jc < a.n ? (float)(jc == a.n - 1 ? a.n_last : a.blk) : -1.0f;
    } else {
      wx_s[tid] = k0 + tid < a.L ? 1.0f : -1.0f;
    }
  }
  __syncthreads();

  f32x16 dk[DT], dv[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dk[dt] = dv[dt] = f32x16{};

  const Rows qrows = tensor_rows(a, a.q, bh), orows = tensor_rows(a, a.dout, bh);
  const size_t row_base = (size_t)bh * a.n * a.blk;
  uint4 pq[PER], po[PER];
  float plse = kInf, pdl = 0.0f;
  unsigned long long pcm = 0ull;
  // item e: query block qlist[e / SPB], 64-row half e % SPB
  auto prefetch = [&](int e) {
    const int i = qlist[e / SPB], r0 = i * a.blk + (e % SPB) * 64;
    load_rows<T, D>(qrows, r0, pq);
    load_rows<T, D>(orows, r0, po);
    if (tid < 64) {
      const int g = r0 + tid;
      plse = g < a.L ? a.lse[row_base + g] : kInf;  // rows past the sequence take no weight
      pdl = g < a.L ? a.delta[row_base + g] : 0.0f;
    }
    if constexpr (CENT) pcm = selected64(a, bh, i, ct);
  };
  for (;;) {
    const int nitems = qcount * SPB, from = qnext;
    if (nitems > 0) prefetch(0);
    for (int e = 0; e < nitems; ++e) {
      __syncthreads();  // q / dO tiles free
      store_rows<T, D>(qt, pq);
      store_rows<T, D>(ot, po);
      if (tid < 64) {
        lse_s[tid] = plse;
        dl_s[tid] = pdl;
      }
      const unsigned long long cmask = pcm;  // centroids the query block selects: no weight
      __syncthreads();
      if (e + 1 < nitems) prefetch(e + 1);
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
        const uint4 pvv = Op<T>::pack(&p[KW * c]);
        const uint4 dsv = Op<T>::pack(&ds[KW * c]);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          Op<T>::mma(dv[dt], pvv, op_col<T, D>(ot, th, dt, c, lane));
          Op<T>::mma(dk[dt], dsv, op_col<T, D>(qt, th, dt, c, lane));
        }
      }
    }
    if (from >= i_hi) break;
    __syncthreads();  // every thread has read qcount, qnext and its last list entry
    list_chunk(from);
    __syncthreads();
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
      const int xx = 32 * xh + vkey(r, h), d = 32 * dt + l32;
      if constexpr (CENT) {
        const int jc = 64 * ct + xx;
        if (a.cparts > 1) {  // raw partial sums, added up by k_bwd_cent_reduce
          const size_t pidx = (((size_t)part * (gridDim.x / a.cparts / a.nct) + bh) * a.nct * 64 + jc) * D + d;
          a.dkbar_p[pidx] = dk[dt][r];
          a.dvsum_p[pidx] = dv[dt][r];
        } else if (jc < a.n) {
          a.dkbar[((size_t)bh * a.n + jc) * D + d] = a.scale * dk[dt][r];
          a.dvsum[((size_t)bh * a.n + jc) * D + d] = dv[dt][r];
        }
      } else {
        const int g = k0 + xx;
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

// The centroid gradients from their partial sums over ranges of query
// blocks, added in range order (deterministic): dk̄_j = s Σ_p part_p.
template <int D>
__global__ void k_bwd_cent_reduce(BwdArgs a, long bh_total) {
  const size_t per = (size_t)bh_total * a.nct * 64 * D;
  for (long x = (long)blockIdx.x * 256 + threadIdx.x; x < bh_total * a.n * D; x += (long)gridDim.x * 256) {
    const long r = x / D;
    const int d = (int)(x % D);
    const long bh = r / a.n;
    const int jc = (int)(r % a.n);
    const size_t o = ((size_t)bh * a.nct * 64 + jc) * D + d;
    float sk = 0.0f, sv = 0.0f;
    for (int p = 0; p < a.cparts; ++p) {
      sk += a.dkbar_p[p * per + o];
      sv += a.dvsum_p[p * per + o];
    }
    a.dkbar[x] = a.scale * sk;
    a.dvsum[x] = sv;
  }
}

// k̄_j and ΣV_j as rows in the I/O dtype (zero past n), for the centroid tiles.
template <typename T, int D>
__global__ void k_bwd_prep(BwdArgs a, long rows) {
  for (long x = (long)blockIdx.x * 256 + threadIdx.x; x < rows * D; x += (long)gridDim.x * 256) {
    const long r = x / D;
    const int d = (int)(x % D);
    const long bh = r / (a.nct * 64);
    const int j = (int)(r % (a.nct * 64));
    const size_t src = ((size_t)bh * a.n + j) * D + d;
    ((T*)a.kbt)[x] = Op<T>::from_f32(j < a.n ? (float)a.kbar[src] : 0.0f);
    ((T*)a.vbt)[x] = Op<T>::from_f32(j < a.n ? (float)a.vsum[src] : 0.0f);
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

__global__ void k_bwd_zero(int* x) { *x = 0; }

// Workgroups of a kernel that can be resident at once, in multiples of the
// eight XCDs (a generation of the XCD-aware order).
template <typename K>
static long resident_wgs(K kernel, long total) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, 0) != hipSuccess)
    return total;
  const long r = (long)(per_cu < 1 ? 1 : per_cu) * cus;
  return r < total ? r : total;
}

template <typename T, int D, int SPB>
hipError_t launch_bwd_t(const BwdArgs& a0, long bh, hipStream_t s) {
  BwdArgs a = a0;
  a.nwg_dq = resident_wgs(k_bwd_dq<T, D, SPB>, a.total);
  a.nwg_dkv = resident_wgs(k_bwd_dkv<T, D, SPB, false>, a.total);
  const size_t words = (size_t)bh * a.n * a.W;
  hipLaunchKernelGGL(k_bwd_selmap_clear, dim3(1024), dim3(256), 0, s, a.selmap, words);
  hipLaunchKernelGGL(k_bwd_selmap_set, dim3((unsigned)(bh * a.n)), dim3(256), 0, s, a);
  const long crow = bh * a.nct * 64;
  hipLaunchKernelGGL((k_bwd_prep<T, D>), dim3((unsigned)min(4096L, (crow * D + 255) / 256)), dim3(256), 0, s, a,
                     crow);
  hipLaunchKernelGGL(k_bwd_zero, dim3(1), dim3(1), 0, s, a.sync);
  hipLaunchKernelGGL((k_bwd_dq<T, D, SPB>), dim3((unsigned)(bh * a.n * SPB)), dim3(256), 0, s, a);
  hipLaunchKernelGGL((k_bwd_dkv<T, D, SPB, true>), dim3((unsigned)(bh * a.nct * a.cparts)), dim3(256), 0, s, a);
  if (a.cparts > 1)
    hipLaunchKernelGGL((k_bwd_cent_reduce<D>), dim3((unsigned)min(4096L, (bh * a.n * D + 255) / 256)), dim3(256), 0,
                       s, a, bh);
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
