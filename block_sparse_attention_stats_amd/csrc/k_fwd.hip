// Fused PISA forward pass (gist.science technical summary of arXiv
// 2602.01077, section 2 "Core Algorithm" N_t equation and "Hardware
// Implementation" phases 1-3; the README's "Kernel variants" for the
// zeroth-order-only form). For query row t of query block i:
//   N_t = Σ_{j∈S_i} Σ_n e^{ℓ_tn} v_n + Σ_{j∈U_i} α_tj ΣV_j + [hyd] A_t · s · q_t H̄
//   D_t = Σ_{j∈S_i} Σ_n e^{ℓ_tn}     + Σ_{j∈U_i} n_j α_tj,
//   ℓ_tn = s q_t·k_n, α_tj = e^{s q_t·k̄_j}, A_t = Σ_{j∈U_i} α_tj,  o_t = N_t / D_t.
// Every exponent of a row is taken relative to one shift m_t, and N_t / D_t
// does not depend on m_t.
//
// Work decomposition (one workgroup = one 64-row query tile, two wavefronts):
//  * each wavefront keeps the whole 64 x D query tile in registers (as MFMA B
//    operands) and a full 64 x D fp32 accumulator Oᵀ, and takes one 32-key
//    half of every 64-key sub-tile (the two halves are summed at the end,
//    which halves each wavefront's K/V traffic);
//  * phase 1, exact: for each selected block (ascending) and each of its 64-key
//    sub-tiles, Sᵀ = K Qᵀ (keys x queries), P = 2^(Sᵀ·s·log2e − m), then
//    Oᵀ += Vᵀ Pᵀ with P taken straight from Sᵀ's registers. K and V come from
//    the operand-ordered copies written by the statistics pass: every operand
//    is one 16-byte load per lane. The next sub-tile's K is loaded into the K
//    registers as soon as Sᵀ has consumed them, its V once Oᵀ has;
//  * phase 2, zeroth order: the centroid tiles k̄ / ΣV are treated as 64-"key"
//    sub-tiles: weights of the selected and padding centroids are zeroed, D
//    gets n_j·p, N gets p·ΣV_j, and A_t accumulates p;
//  * phase 3, first order: Uᵀ = H̄ᵀ Qᵀ on MFMA after the halves are summed,
//    N += A_t · s · Uᵀ; then o = N / D.
//
// The shift. Every logit obeys s q_t·k ≤ s ‖q_t‖ max‖k‖ (Cauchy–Schwarz; a
// centroid's norm is at most the largest key norm), so with
// m_t = s log2(e) ‖q_t‖ max‖k‖ − 64 no weight exceeds 2^64 and the fast kernel
// needs no running maximum and never rescales its accumulators. If the bound is
// so loose that a row's denominator falls below 2^-60 (its weights would lose
// precision near the bottom of the fp32 range), the fast kernel leaves the
// tile to k_pisa_fwd_careful, which recomputes it with the classic running
// maximum (raised whenever a row max grows by more than 2^8).
#include "pisa_dev.h"
#include "pisa_internal.h"

namespace pisa {

namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kHeadroom = 64.0f;      // log2 headroom between the logit bound and the shift
constexpr float kTinyDenom = 0x1p-60f;  // below this a tile goes to the careful kernel
constexpr float kTau = 8.0f;            // careful kernel: log2 growth that raises the max

enum TileKind { kExactFull = 0, kExactRagged = 1, kCentroid = 2 };

// Register-array types of one wavefront's state.
template <typename T, int D>
struct Regs {
  using G = Geo<T, D>;
  typedef uint4 Q[2][G::NC];               // query tile as B operands
  typedef f32x16 Acc[G::DT][2];            // Oᵀ accumulators (d x query)
  typedef uint4 K[G::NC];                  // K-format operands of one 32-key half
  typedef uint4 V[G::DT * G::CPK];         // V-format operands of one 32-key half
  typedef uint4 P[2][G::CPK];              // softmax weights as B operands
  typedef float Xo[2][G::DT / 2][2][16][kWave];  // LDS exchange of accumulator halves
};

struct FwdShared {
  uint32_t selmask[kMaxBlocks / 32];
  float xstat[2][3][2][32];
};

template <typename T, int D>
__device__ __forceinline__ void load_k(const uint8_t* tile, int w, int lane,
                                       typename Regs<T, D>::K& kc) {
  using G = Geo<T, D>;
#pragma unroll
  for (int c = 0; c < G::NC; ++c) kc[c] = *(const uint4*)(tile + ((w * G::NC + c) * kWave + lane) * 16);
}

template <typename T, int D>
__device__ __forceinline__ void load_v(const uint8_t* tile, int w, int lane,
                                       typename Regs<T, D>::V& vc) {
  using G = Geo<T, D>;
  constexpr int NV = G::DT * G::CPK;
#pragma unroll
  for (int x = 0; x < NV; ++x) vc[x] = *(const uint4*)(tile + ((w * NV + x) * kWave + lane) * 16);
}

template <typename T, int D>
__device__ __forceinline__ void mma_s(const typename Regs<T, D>::Q& qr,
                                      const typename Regs<T, D>::K& kc, f32x16 (&sacc)[2]) {
  using G = Geo<T, D>;
  sacc[0] = f32x16{};
  sacc[1] = f32x16{};
#pragma unroll
  for (int c = 0; c < G::NC; ++c) {
    Op<T>::mma(sacc[0], kc[c], qr[0][c]);
    Op<T>::mma(sacc[1], kc[c], qr[1][c]);
  }
}

template <typename T, int D>
__device__ __forceinline__ void mma_pv(typename Regs<T, D>::Acc& oacc,
                                       const typename Regs<T, D>::V& vc,
                                       const typename Regs<T, D>::P& pc) {
  using G = Geo<T, D>;
#pragma unroll
  for (int dt = 0; dt < G::DT; ++dt)
#pragma unroll
    for (int c = 0; c < G::CPK; ++c) {
      Op<T>::mma(oacc[dt][0], vc[dt * G::CPK + c], pc[0][c]);
      Op<T>::mma(oacc[dt][1], vc[dt * G::CPK + c], pc[1][c]);
    }
}

// Is accumulator register r of lane half h outside the tile (key 32*w + vkey
// beyond `valid`) or, for centroids, a selected block?
template <int KIND>
__device__ __forceinline__ bool dead_key(int r, int h, int w, int valid, uint32_t selword) {
  if constexpr (KIND == kExactFull) return false;
  const int kk = vkey(r, h);
  bool dead = (32 * w + kk) >= valid;
  if constexpr (KIND == kCentroid) dead = dead || ((selword >> kk) & 1u);
  return dead;
}

// Weights P = 2^(Sᵀ·cs − m) of one sub-tile, the row sums (D gets n_j per
// centroid) and the P operands.
template <typename T, int D, int KIND>
__device__ __forceinline__ void tile_weights(const f32x16 (&sacc)[2], const float (&m)[2],
                                             float (&l)[2], float (&asum)[2],
                                             typename Regs<T, D>::P& pc, float cs, int h, int w,
                                             int valid, uint32_t selword, int klast, float blk_w,
                                             float last_w) {
  using G = Geo<T, D>;
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const float ms = (m[qt] == kNegInf) ? 0.0f : m[qt];
    float p[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      p[r] = __builtin_amdgcn_exp2f(fmaf(sacc[qt][r], cs, -ms));
      if constexpr (KIND != kExactFull) p[r] = dead_key<KIND>(r, h, w, valid, selword) ? 0.0f : p[r];
    }
    float ps = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) ps += p[r];
    if constexpr (KIND == kCentroid) {
      // D gets n_j per centroid: the block size, except for the last block
      float wsum = ps * blk_w;
#pragma unroll
      for (int r = 0; r < 16; ++r) wsum += (vkey(r, h) == klast) ? p[r] * last_w : 0.0f;
      l[qt] += wsum;
      asum[qt] += ps;
    } else {
      l[qt] += ps;
    }
#pragma unroll
    for (int c = 0; c < G::CPK; ++c) pc[qt][c] = Op<T>::pack(&p[G::KW * c]);
  }
}

// Careful kernel only: does any row of this sub-tile need a higher running max?
template <int KIND>
__device__ __forceinline__ bool tile_max(const f32x16 (&sacc)[2], const float (&m)[2],
                                         float (&mt)[2], bool (&need)[2], float cs, int h, int w,
                                         int valid, uint32_t selword) {
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    float mx = kNegInf;
#pragma unroll
    for (int r = 0; r < 16; ++r)
      mx = fmaxf(mx, dead_key<KIND>(r, h, w, valid, selword) ? kNegInf : sacc[qt][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    mt[qt] = mx * cs;
    need[qt] = mt[qt] > m[qt] + kTau;
  }
  return __any(need[0] || need[1]);
}

template <typename T, int D>
__device__ __forceinline__ void raise_max(typename Regs<T, D>::Acc& oacc, float (&m)[2],
                                          float (&l)[2], float (&asum)[2], const float (&mt)[2],
                                          const bool (&need)[2]) {
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const float mn = need[qt] ? mt[qt] : m[qt];
    const float alpha = need[qt] ? __builtin_amdgcn_exp2f(m[qt] - mn) : 1.0f;
    m[qt] = mn;
    l[qt] *= alpha;
    asum[qt] *= alpha;
#pragma unroll
    for (int dt = 0; dt < Geo<T, D>::DT; ++dt) oacc[dt][qt] *= alpha;
  }
}

// One sub-tile: Sᵀ, weights, Oᵀ += Vᵀ Pᵀ, with the next sub-tile's K and V
// loads issued as soon as their registers are free.
template <typename T, int D, bool CAREFUL, int KIND>
__device__ __forceinline__ void step(typename Regs<T, D>::Acc& oacc, const typename Regs<T, D>::Q& qr,
                                     typename Regs<T, D>::K& kc, typename Regs<T, D>::V& vc,
                                     float (&m)[2], float (&l)[2], float (&asum)[2], float cs,
                                     int h, int w, int lane, int valid, uint32_t selword, int klast,
                                     float blk_w, float last_w, const uint8_t* knext,
                                     const uint8_t* vnext) {
  f32x16 sacc[2];
  typename Regs<T, D>::P pc;
  mma_s<T, D>(qr, kc, sacc);
  if (knext) load_k<T, D>(knext, w, lane, kc);
  if constexpr (CAREFUL) {
    float mt[2];
    bool need[2];
    if (tile_max<KIND>(sacc, m, mt, need, cs, h, w, valid, selword))
      raise_max<T, D>(oacc, m, l, asum, mt, need);
  }
  tile_weights<T, D, KIND>(sacc, m, l, asum, pc, cs, h, w, valid, selword, klast, blk_w, last_w);
  mma_pv<T, D>(oacc, vc, pc);
  if (vnext) load_v<T, D>(vnext, w, lane, vc);
}

// Sums the two wavefronts' partial states (wavefront W finishes output tiles
// W*DH .. W*DH+DH-1), adds the first-order term and stores o = N / D. In the
// fast kernel a tile whose denominator is too small is queued for the careful
// kernel and nothing is stored.
template <typename T, int D, bool CAREFUL, int W>
__device__ __forceinline__ void epilogue(const FwdArgs& a, typename Regs<T, D>::Acc& oacc,
                                         float (&m)[2], float (&l)[2], float (&asum)[2],
                                         const typename Regs<T, D>::Q& qr, FwdShared& sh,
                                         typename Regs<T, D>::Xo& xo, bool tail, long bh, int r0,
                                         int lane, long item) {
  using G = Geo<T, D>;
  using O = Op<T>;
  constexpr int NC = G::NC, DT = G::DT, ESZ = G::ESZ;
  constexpr int DH = DT / 2;
  constexpr int w = W;
  const int h = lane >> 5, l32 = lane & 31;
  float Lt[2], At[2];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const float lt = l[qt] + __shfl_xor(l[qt], 32);
    const float at = asum[qt] + __shfl_xor(asum[qt], 32);
    if (h == 0) {
      sh.xstat[w][0][qt][l32] = m[qt];
      sh.xstat[w][1][qt][l32] = lt;
      sh.xstat[w][2][qt][l32] = at;
    }
    l[qt] = lt;
    asum[qt] = at;
  }
#pragma unroll
  for (int t = 0; t < DH; ++t)
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
      for (int r = 0; r < 16; ++r) xo[w][t][qt][r][lane] = oacc[(1 - w) * DH + t][qt][r];
  __syncthreads();
  bool tiny = false;
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const float mp = sh.xstat[1 - w][0][qt][l32];
    const float lp = sh.xstat[1 - w][1][qt][l32];
    const float ap = sh.xstat[1 - w][2][qt][l32];
    float fs = 1.0f, fp = 1.0f;  // the fast kernel's shift is the same in both wavefronts
    if constexpr (CAREFUL) {
      const float mstar = fmaxf(m[qt], mp);
      fs = (m[qt] == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(m[qt] - mstar);
      fp = (mp == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(mp - mstar);
    }
    Lt[qt] = fs * l[qt] + fp * lp;
    At[qt] = fs * asum[qt] + fp * ap;
    const int row = r0 + 32 * qt + l32;
    if (!CAREFUL && row < a.L && !(Lt[qt] >= kTinyDenom && Lt[qt] < __builtin_huge_valf())) tiny = true;
#pragma unroll
    for (int t = 0; t < DH; ++t) {
      const int dt = w * DH + t;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        oacc[dt][qt][r] = fs * oacc[dt][qt][r] + fp * xo[1 - w][t][qt][r][lane];
    }
  }
  if constexpr (!CAREFUL) {
    // both wavefronts see the same sums, hence the same verdict
    if (__any(tiny)) {
      if (w == 0 && lane == 0) {
        const int slot = atomicAdd(a.redo, 1);
        a.redo[1 + slot] = (int)item;
      }
      return;
    }
  }

  // ---- phase 3: global first-order correction A_t · s · q_t H̄
  if (tail && a.first_order) {
    const uint8_t* hb = a.hbt + (size_t)bh * D * D * ESZ;
#pragma unroll
    for (int t = 0; t < DH; ++t) {
      const int et = w * DH + t;
      f32x16 u[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const uint4 hc = *(const uint4*)(hb + ((et * NC + c) * kWave + lane) * 16);
        O::mma(u[0], hc, qr[0][c]);
        O::mma(u[1], hc, qr[1][c]);
      }
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) oacc[et][qt] += (At[qt] * a.scale) * u[qt];
    }
  }

  // ---- o = N / D
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int row = r0 + 32 * qt + l32;
    if (row >= a.L) continue;
    const float inv = 1.0f / Lt[qt];
#pragma unroll
    for (int t = 0; t < DH; ++t) {
      const int dt = w * DH + t;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * dt + 8 * g + 4 * h;
        T ov[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[e] = O::from_f32(oacc[dt][qt][4 * g + e] * inv);
        uint8_t* dst = a.o + (((size_t)bh * a.L + row) * D + d) * ESZ;
        if constexpr (ESZ == 2)
          *(uint2*)dst = __builtin_bit_cast(uint2, ov);
        else
          *(uint4*)dst = __builtin_bit_cast(uint4, ov);
      }
    }
  }
}

// The whole forward pass of one 64-row query tile (`item` = (bh, query block,
// 64-row half of a 128-row block)).
template <typename T, int D, bool CAREFUL>
__device__ __forceinline__ void query_tile(const FwdArgs& a, long item, FwdShared& sh,
                                           typename Regs<T, D>::Xo& xo) {
  using G = Geo<T, D>;
  constexpr int NC = G::NC, DT = G::DT, ESZ = G::ESZ, KW = G::KW;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, l32 = lane & 31;
  const int spb = a.blk / kSub;
  const int half = (int)(item % spb);
  const long rest = item / spb;
  const int i = (int)(rest % a.n);
  const long bh = rest / a.n;
  const int r0 = i * a.blk + half * kSub;
  if (r0 >= a.L) return;

  const bool dense = (a.idx == nullptr);
  const int nsel = dense ? a.n : a.topk;
  const int32_t* myidx = dense ? nullptr : a.idx + (bh * a.n + i) * (long)a.topk;
  const bool tail = a.tail && !dense && nsel < a.n;
  // indices outside [0, n) are clamped: a bad selection cannot read out of bounds
  auto block_at = [&](int s) { return dense ? s : min(max(myidx[s], 0), a.n - 1); };

  if (tail) {
    const int nw = (a.n + 31) >> 5;
    for (int x = tid; x < nw; x += 128) sh.selmask[x] = 0u;
    __syncthreads();
    for (int s = tid; s < nsel; s += 128) {
      const int j = block_at(s);
      atomicOr(&sh.selmask[j >> 5], 1u << (j & 31));
    }
    __syncthreads();
  }

  typename Regs<T, D>::Q qr;
  typename Regs<T, D>::Acc oacc;
  float m[2], l[2], asum[2];
  const float cs = a.cs;
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int row = r0 + 32 * qt + l32;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int d0 = 2 * KW * c + KW * h;
      qr[qt][c] = row < a.L ? *(const uint4*)(a.q + (((size_t)bh * a.L + row) * D + d0) * ESZ)
                            : make_uint4(0, 0, 0, 0);
    }
    l[qt] = 0.f;
    asum[qt] = 0.f;
  }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt][0] = oacc[dt][1] = f32x16{};

  if constexpr (CAREFUL) {
    m[0] = m[1] = kNegInf;
  } else {
    // m_t = s log2(e) ‖q_t‖ max‖k‖ − 64
    float qn2[2] = {0.f, 0.f};
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        T e[KW];
        __builtin_memcpy(e, &qr[qt][c], 16);
#pragma unroll
        for (int x = 0; x < KW; ++x) {
          const float f = Op<T>::to_f32(e[x]);
          qn2[qt] = fmaf(f, f, qn2[qt]);
        }
      }
    float km = 0.f;
    for (int c = lane; c < a.nch; c += kWave) km = fmaxf(km, a.kmax2[bh * a.nch + c]);
    km = wave_max(km);
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const float q2 = qn2[qt] + __shfl_xor(qn2[qt], 32);
      m[qt] = cs * sqrtf(q2 * km) - kHeadroom;
    }
  }

  typename Regs<T, D>::K kc;
  typename Regs<T, D>::V vc;

  // ---- phase 1: exact selected blocks, ascending
  {
    const size_t head_sub = (size_t)bh * a.n * spb;
    const int nsub_last = (a.n_last + kSub - 1) / kSub;
    int s = 0, st = 0;
    int j = block_at(0);
    load_k<T, D>(a.kp + (head_sub + (size_t)j * spb) * G::SUB_BYTES, w, lane, kc);
    load_v<T, D>(a.vp + (head_sub + (size_t)j * spb) * G::SUB_BYTES, w, lane, vc);
    while (true) {
      const bool lastblk = (j == a.n - 1);
      const int valid = lastblk ? min(kSub, a.n_last - kSub * st) : kSub;
      int s2 = s, st2 = st + 1, j2 = j;
      if (st2 >= (lastblk ? nsub_last : spb)) {
        s2 = s + 1;
        st2 = 0;
        j2 = (s2 < nsel) ? block_at(s2) : 0;
      }
      const bool more = s2 < nsel;
      const size_t sub2 = head_sub + (size_t)j2 * spb + st2;
      const uint8_t* kn = more ? a.kp + sub2 * G::SUB_BYTES : nullptr;
      const uint8_t* vn = more ? a.vp + sub2 * G::SUB_BYTES : nullptr;
      if (valid == kSub)
        step<T, D, CAREFUL, kExactFull>(oacc, qr, kc, vc, m, l, asum, cs, h, w, lane, valid, 0u,
                                        -1, 0.f, 0.f, kn, vn);
      else
        step<T, D, CAREFUL, kExactRagged>(oacc, qr, kc, vc, m, l, asum, cs, h, w, lane, valid, 0u,
                                          -1, 0.f, 0.f, kn, vn);
      if (!more) break;
      s = s2;
      st = st2;
      j = j2;
    }
  }

  // ---- phase 2: zeroth-order terms of the unselected blocks
  if (tail) {
    const size_t head_ct = (size_t)bh * a.nct;
    const float blk_w = (float)a.blk, last_w = (float)(a.n_last - a.blk);
    load_k<T, D>(a.kbp + head_ct * G::SUB_BYTES, w, lane, kc);
    load_v<T, D>(a.vbp + head_ct * G::SUB_BYTES, w, lane, vc);
    for (int ct = 0; ct < a.nct; ++ct) {
      const bool more = ct + 1 < a.nct;
      const int jbase = kSub * ct + 32 * w;
      const uint32_t word = sh.selmask[jbase >> 5];
      const size_t nxt = (head_ct + ct + 1) * G::SUB_BYTES;
      step<T, D, CAREFUL, kCentroid>(oacc, qr, kc, vc, m, l, asum, cs, h, w, lane, a.n - kSub * ct,
                                     word, a.n - 1 - jbase, blk_w, last_w,
                                     more ? a.kbp + nxt : nullptr, more ? a.vbp + nxt : nullptr);
    }
  }

  // ---- merge, first-order term, output (wave-uniform branch: every register
  // index is a compile-time constant)
  if (w == 0)
    epilogue<T, D, CAREFUL, 0>(a, oacc, m, l, asum, qr, sh, xo, tail, bh, r0, lane, item);
  else
    epilogue<T, D, CAREFUL, 1>(a, oacc, m, l, asum, qr, sh, xo, tail, bh, r0, lane, item);
}

}  // namespace

template <typename T, int D>
__global__ __launch_bounds__(128, 1) void k_pisa_fwd(FwdArgs a) {
  __shared__ FwdShared sh;
  __shared__ typename Regs<T, D>::Xo xo;
  long item;
  if (a.map_mode == 1) {
    item = xcd_remap(blockIdx.x, a.total, a.per_xcd);
  } else {
    item = blockIdx.x;
    if (item >= a.total) item = -1;
  }
  if (item < 0) return;
  query_tile<T, D, false>(a, item, sh, xo);
}

// Recomputes, with a running maximum, the query tiles the fast kernel queued.
template <typename T, int D>
__global__ __launch_bounds__(128, 1) void k_pisa_fwd_careful(FwdArgs a) {
  __shared__ FwdShared sh;
  __shared__ typename Regs<T, D>::Xo xo;
  const int count = *(volatile int*)a.redo;
  for (int e = blockIdx.x; e < count; e += gridDim.x) {
    const long item = a.redo[1 + e];
    __syncthreads();  // shared state of the previous tile fully consumed
    query_tile<T, D, true>(a, item, sh, xo);
  }
}

__global__ void k_zero_counter(int* p) { *p = 0; }

template <typename T, int D>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_zero_counter, dim3(1), dim3(1), 0, s, a.redo);
  const long grid = a.map_mode == 1 ? a.per_xcd * kNumXcd : a.total;
  hipLaunchKernelGGL((k_pisa_fwd<T, D>), dim3((unsigned)grid), dim3(128), 0, s, a);
  hipLaunchKernelGGL((k_pisa_fwd_careful<T, D>), dim3(256), dim3(128), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fwd(int dtype, int D, const FwdArgs& a, hipStream_t s) {
  if (dtype == 1) return D == 64 ? launch_fwd_t<bf16, 64>(a, s) : launch_fwd_t<bf16, 128>(a, s);
  return D == 64 ? launch_fwd_t<float, 64>(a, s) : launch_fwd_t<float, 128>(a, s);
}

}  // namespace pisa
