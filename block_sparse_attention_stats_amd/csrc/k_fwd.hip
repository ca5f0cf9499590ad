// Fused PISA forward pass (gist.science technical summary of arXiv
// 2602.01077, section 2 "Core Algorithm" N_t equation and "Hardware
// Implementation" phases 1-3; the README's "Kernel variants" for the
// zeroth-order-only form). For query row t of query block i:
//   N_t = Σ_{j∈S_i} Σ_n e^{ℓ_tn} v_n + Σ_{j∈U_i} α_tj ΣV_j + [hyd] A_t · s · q_t H̄
//   D_t = Σ_{j∈S_i} Σ_n e^{ℓ_tn}     + Σ_{j∈U_i} n_j α_tj,
//   ℓ_tn = s q_t·k_n, α_tj = e^{s q_t·k̄_j}, A_t = Σ_{j∈U_i} α_tj,  o_t = N_t / D_t,
// all inside one online softmax (every exponent shares the running maximum).
//
// Work decomposition (one workgroup = one 64-row query tile, two wavefronts):
//  * each wavefront keeps the whole 64 x D query tile in registers (as MFMA B
//    operands) and a full 64 x D fp32 accumulator Oᵀ, and takes one 32-key
//    half of every 64-key sub-tile ("split-K": the two partial softmax states
//    are merged at the end, which halves each wavefront's K/V traffic);
//  * phase 1, exact: for each selected block (ascending) and each of its 64-key
//    sub-tiles, Sᵀ = K Qᵀ (keys x queries), online softmax in registers (the
//    row of a lane pair l, l^32 is one query, so a row max is one lane swap),
//    then Oᵀ += Vᵀ Pᵀ with P taken straight from Sᵀ's registers. K and V come
//    from the operand-ordered copies written by the statistics pass: every
//    operand is one 16-byte load per lane, the next sub-tile's loads are in
//    flight while the current one is computed;
//  * phase 2, zeroth order: the centroid tiles k̄ / ΣV are treated as 64-"key"
//    sub-tiles: logits s q·k̄_j (selected and padding columns masked) join the
//    same running max, D gets n_j·p, N gets p·ΣV_j, and A_t accumulates p;
//  * phase 3, first order: Uᵀ = H̄ᵀ Qᵀ on MFMA after the two halves are merged,
//    N += A_t · s · Uᵀ; then o = N / D.
// The running max is only raised when a row's max grows by more than 2^8
// (weights stay ≤ 256, far inside fp32 and bf16 range), so the accumulator is
// rarely rescaled.
#include "pisa_dev.h"
#include "pisa_internal.h"

namespace pisa {

template <typename T, int D>
__global__ __launch_bounds__(128, 1) void k_pisa_fwd(FwdArgs a) {
  using G = Geo<T, D>;
  using O = Op<T>;
  constexpr int KW = G::KW, NC = G::NC, DT = G::DT, CPK = G::CPK, ESZ = G::ESZ;
  constexpr int DH = DT / 2;  // output tiles finished by each wavefront
  constexpr float TAU = 8.0f;
  constexpr float NEG_INF = -__builtin_huge_valf();

  __shared__ uint32_t selmask[kMaxBlocks / 32];
  __shared__ float xstat[2][3][2][32];
  __shared__ float xo[2][DH][2][16][kWave];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, l32 = lane & 31;
  const long item = xcd_remap(blockIdx.x, a.total, a.per_xcd);
  if (item < 0) return;
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

  if (tail) {
    const int nw = (a.n + 31) >> 5;
    for (int x = tid; x < nw; x += 128) selmask[x] = 0u;
    __syncthreads();
    for (int s = tid; s < nsel; s += 128) {
      const int j = min(max(myidx[s], 0), a.n - 1);
      atomicOr(&selmask[j >> 5], 1u << (j & 31));
    }
    __syncthreads();
  }

  // Query tile as B operands: qr[qt][c] = row r0+32qt+l32, d = 2KW c + KW h ...
  uint4 qr[2][NC];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int row = r0 + 32 * qt + l32;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int d0 = 2 * KW * c + KW * h;
      qr[qt][c] = row < a.L ? *(const uint4*)(a.q + (((size_t)bh * a.L + row) * D + d0) * ESZ)
                            : make_uint4(0, 0, 0, 0);
    }
  }

  f32x16 oacc[DT][2];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt][0] = oacc[dt][1] = f32x16{};
  float m[2] = {NEG_INF, NEG_INF}, l[2] = {0.f, 0.f}, asum[2] = {0.f, 0.f};
  const float cs = a.cs;

  // One 64-key sub-tile: this wavefront's 32 keys. mode 0 = exact keys, 1 = centroids.
  auto process = [&](const uint4 (&kc)[NC], const uint4 (&vc)[DT * CPK], int mode, int valid,
                     uint32_t selword, int jbase) {
    f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      O::mma(sacc[0], kc[c], qr[0][c]);
      O::mma(sacc[1], kc[c], qr[1][c]);
    }
    // masks: keys beyond `valid`; for centroids also the selected blocks
    if (mode == 1 || valid < kSub) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = vkey(r, h);  // key within this wavefront's 32
        bool dead = (32 * w + kk) >= valid;
        if (mode == 1) dead = dead || ((selword >> kk) & 1u);
        if (dead) {
          sacc[0][r] = NEG_INF;
          sacc[1][r] = NEG_INF;
        }
      }
    }
    float mt[2];
    bool need[2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      float mx = sacc[qt][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sacc[qt][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      mt[qt] = mx * cs;
      need[qt] = mt[qt] > m[qt] + TAU;
    }
    if (__any(need[0] || need[1])) {
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        const float mn = need[qt] ? mt[qt] : m[qt];
        const float alpha = need[qt] ? __builtin_amdgcn_exp2f(m[qt] - mn) : 1.0f;
        m[qt] = mn;
        l[qt] *= alpha;
        asum[qt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) oacc[dt][qt] *= alpha;
      }
    }
    uint4 pc[2][CPK];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const float ms = (m[qt] == NEG_INF) ? 0.0f : m[qt];
      float p[16];
      float ps = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[r] = __builtin_amdgcn_exp2f(fmaf(sacc[qt][r], cs, -ms));
        ps += p[r];
      }
      if (mode == 0) {
        l[qt] += ps;
      } else {
        // D gets n_j per centroid: block size everywhere but the last block
        float wsum = ps * (float)a.blk;
        const int klast = a.n - 1 - jbase;  // position of the last block in this 32
        if (klast >= 0 && klast < 32) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (vkey(r, h) == klast) wsum += p[r] * (float)(a.n_last - a.blk);
        }
        l[qt] += wsum;
        asum[qt] += ps;
      }
#pragma unroll
      for (int c = 0; c < CPK; ++c) pc[qt][c] = O::pack(&p[KW * c]);
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int c = 0; c < CPK; ++c) {
        O::mma(oacc[dt][0], vc[dt * CPK + c], pc[0][c]);
        O::mma(oacc[dt][1], vc[dt * CPK + c], pc[1][c]);
      }
  };

  auto load_tiles = [&](const uint8_t* kt, const uint8_t* vt, uint4 (&kc)[NC],
                        uint4 (&vc)[DT * CPK]) {
#pragma unroll
    for (int c = 0; c < NC; ++c) kc[c] = *(const uint4*)(kt + ((w * NC + c) * kWave + lane) * 16);
#pragma unroll
    for (int x = 0; x < DT * CPK; ++x) vc[x] = *(const uint4*)(vt + ((w * DT * CPK + x) * kWave + lane) * 16);
  };

  // ---- phase 1: exact selected blocks
  const size_t head_sub = (size_t)bh * a.n * spb;
  const int nsub_last = (a.n_last + kSub - 1) / kSub;
  if (nsel > 0) {
    int s = 0, st = 0;
    // indices outside [0, n) are clamped: a bad selection cannot read out of bounds
    auto block_at = [&](int s) { return dense ? s : min(max(myidx[s], 0), a.n - 1); };
    int j = block_at(0);
    uint4 kc[NC], vc[DT * CPK];
    load_tiles(a.kp + (head_sub + (size_t)j * spb) * G::SUB_BYTES,
               a.vp + (head_sub + (size_t)j * spb) * G::SUB_BYTES, kc, vc);
    while (s < nsel) {
      const bool lastblk = (j == a.n - 1);
      const int valid = lastblk ? min(kSub, a.n_last - kSub * st) : kSub;
      int s2 = s, st2 = st + 1, j2 = j;
      if (st2 >= (lastblk ? nsub_last : spb)) {
        s2 = s + 1;
        st2 = 0;
        j2 = (s2 < nsel) ? block_at(s2) : 0;
      }
      uint4 kn[NC], vn[DT * CPK];
      if (s2 < nsel) {
        const size_t sub = head_sub + (size_t)j2 * spb + st2;
        load_tiles(a.kp + sub * G::SUB_BYTES, a.vp + sub * G::SUB_BYTES, kn, vn);
      }
      process(kc, vc, 0, valid, 0u, 0);
#pragma unroll
      for (int c = 0; c < NC; ++c) kc[c] = kn[c];
#pragma unroll
      for (int x = 0; x < DT * CPK; ++x) vc[x] = vn[x];
      s = s2;
      st = st2;
      j = j2;
    }
  }

  // ---- phase 2: zeroth-order terms of the unselected blocks
  if (tail) {
    const size_t head_ct = (size_t)bh * a.nct;
    uint4 kc[NC], vc[DT * CPK];
    load_tiles(a.kbp + head_ct * G::SUB_BYTES, a.vbp + head_ct * G::SUB_BYTES, kc, vc);
    for (int ct = 0; ct < a.nct; ++ct) {
      uint4 kn[NC], vn[DT * CPK];
      if (ct + 1 < a.nct)
        load_tiles(a.kbp + (head_ct + ct + 1) * G::SUB_BYTES,
                   a.vbp + (head_ct + ct + 1) * G::SUB_BYTES, kn, vn);
      const int jbase = kSub * ct + 32 * w;
      const uint32_t word = selmask[jbase >> 5];
      process(kc, vc, 1, a.n - kSub * ct, word, jbase);
#pragma unroll
      for (int c = 0; c < NC; ++c) kc[c] = kn[c];
#pragma unroll
      for (int x = 0; x < DT * CPK; ++x) vc[x] = vn[x];
    }
  }

  // ---- merge the two wavefronts' softmax states
  float Lt[2], At[2];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const float lt = l[qt] + __shfl_xor(l[qt], 32);
    const float at = asum[qt] + __shfl_xor(asum[qt], 32);
    if (h == 0) {
      xstat[w][0][qt][l32] = m[qt];
      xstat[w][1][qt][l32] = lt;
      xstat[w][2][qt][l32] = at;
    }
    l[qt] = lt;
    asum[qt] = at;
  }
  __syncthreads();
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const float mp = xstat[1 - w][0][qt][l32];
    const float lp = xstat[1 - w][1][qt][l32];
    const float ap = xstat[1 - w][2][qt][l32];
    const float mstar = fmaxf(m[qt], mp);
    const float fs = (m[qt] == NEG_INF) ? 0.0f : __builtin_amdgcn_exp2f(m[qt] - mstar);
    const float fp = (mp == NEG_INF) ? 0.0f : __builtin_amdgcn_exp2f(mp - mstar);
    Lt[qt] = fs * l[qt] + fp * lp;
    At[qt] = fs * asum[qt] + fp * ap;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt][qt] *= fs;
  }
#pragma unroll
  for (int t = 0; t < DH; ++t)
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
      for (int r = 0; r < 16; ++r) xo[w][t][qt][r][lane] = oacc[(1 - w) * DH + t][qt][r];
  __syncthreads();
#pragma unroll
  for (int t = 0; t < DH; ++t)
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[w * DH + t][qt][r] += xo[1 - w][t][qt][r][lane];

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
    if (row >= a.L || row >= (i + 1) * a.blk) continue;
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

template <typename T, int D>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t s) {
  dim3 grid((unsigned)(a.per_xcd * kNumXcd));
  hipLaunchKernelGGL((k_pisa_fwd<T, D>), grid, dim3(128), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fwd(int dtype, int D, const FwdArgs& a, hipStream_t s) {
  if (dtype == 1) return D == 64 ? launch_fwd_t<bf16, 64>(a, s) : launch_fwd_t<bf16, 128>(a, s);
  return D == 64 ? launch_fwd_t<float, 64>(a, s) : launch_fwd_t<float, 128>(a, s);
}

}  // namespace pisa
