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
// With a fixed shift the order of phases 1 and 2 is free: short exact sweeps
// scan the centroids first, long ones last (query_tile). Workgroups run in
// generations of as many as are resident, and each lines up its exact sweep
// with the others of its generation (k_pisa_fwd), so gathered blocks are
// reused from the L2. For bf16 the sub-tile loop is written out in issue order
// (xstep), since one wavefront per SIMD only overlaps MFMA and VALU work where
// the instruction stream alternates them.
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
constexpr int kCentroidsFirstBelow = 96;  // exact sub-tiles below which the centroid scan goes first
constexpr int kEarlySignalMaxCt = 24;     // centroid tiles up to which a workgroup counts as done
                                          // for the generation wait once its exact sweep ends

enum TileKind { kExactFull = 0, kExactRagged = 1, kCentroid = 2 };

// Address of token `row` of head bh in q (OUT false) or o (OUT true): either
// layout, and either part of a sequence held in two tensors.
template <bool OUT>
__device__ __forceinline__ auto io_row(const FwdArgs& a, long bh, int row) {
  const long b = bh / a.H, h = bh % a.H;
  if (row < a.L0) {
    const size_t off = (size_t)b * a.stride_b + (size_t)h * a.stride_h + (size_t)row * a.stride_l;
    if constexpr (OUT) return a.o + off; else return a.q + off;
  }
  // The second part's fields are loaded here, where they are used, from the
  // kernel's argument segment (every kernel calling this takes one FwdArgs
  // and nothing else), rather than held in scalar registers through the
  // whole kernel. (A volatile reference to the argument itself would copy the
  // struct to scratch memory.)
  using kargs_t = const volatile FwdArgs __attribute__((address_space(4)));
  kargs_t* v = (kargs_t*)__builtin_amdgcn_kernarg_segment_ptr();
  const size_t off = (size_t)b * v->stride1_b + (size_t)h * v->stride1_h + (size_t)(row - a.L0) * v->stride1_l;
  if constexpr (OUT) return (uint8_t*)v->o1 + off; else return (const uint8_t*)v->q1 + off;
}

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

template <typename T, int D>
struct FwdShared {
  uint32_t selmask[kMaxBlocks / 32];  // selected blocks of the query tile, one bit each
  float xstat[2][3][2][32];           // per-wavefront row statistics exchanged at the merge
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

// Sᵀ = K Qᵀ for the two 32-row query tiles, accumulated onto `init` (zeros, or
// −inf at keys that must get no weight).
template <typename T, int D>
__device__ __forceinline__ void mma_s(const typename Regs<T, D>::Q& qr,
                                      const typename Regs<T, D>::K& kc, f32x16 (&sacc)[2],
                                      const f32x16& init = f32x16{}) {
  using G = Geo<T, D>;
  sacc[0] = init;
  sacc[1] = init;
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
#pragma unroll
    for (int c = 0; c < G::CPK; ++c) {
      pc[qt][c] = Op<T>::pack(&p[G::KW * c]);
      Op<T>::unpack(pc[qt][c], &p[G::KW * c]);  // the sums take the rounded weights
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
  }
}

// Weights of a full sub-tile: P = 2^(Sᵀ·cs − m) and its row sums. The
// numerator takes P rounded to the operand type. With RSUM the sums take the
// rounded values too (unpacked with two bit operations per pair), so that a
// row whose weight sits on one key returns that key's value exactly; the
// exact sweeps use it. The centroid scan keeps fp32 sums, which the fast
// kernel's correction for the short last block (an fp32 weight recomputed in
// the epilogue, times n_last − blk) must match. The written-out main loop
// (xstep) sums fp32 values, as unbiased, and saves those operations where it
// counts; a sweep's first and last tiles always come here.
template <typename T, int D, bool RSUM>
__device__ __forceinline__ void weights_full(const f32x16 (&sacc)[2], const float (&m)[2],
                                             float (&l)[2], typename Regs<T, D>::P& pc, float cs) {
  using G = Geo<T, D>;
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
#pragma unroll
    for (int c = 0; c < G::CPK; ++c) {
      float p[G::KW];
#pragma unroll
      for (int e = 0; e < G::KW; ++e)
        p[e] = __builtin_amdgcn_exp2f(fmaf(sacc[qt][G::KW * c + e], cs, -m[qt]));
      pc[qt][c] = Op<T>::pack(p);
      if constexpr (RSUM) Op<T>::unpack(pc[qt][c], p);
#pragma unroll
      for (int e = 0; e < G::KW; e += 2) l[qt] += p[e] + p[e + 1];
    }
  }
}

// Scheduling hint for one pipelined tile of fp32 operands (bf16 uses xstep):
// alternate the MFMAs of PV(t) and Sᵀ(t+2) with the VALU work of P(t+1),
// spreading the loads among them.
__device__ __forceinline__ void interleave_tile() {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // VALU
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // VALU
  }
}

// One software-pipelined sub-tile for bf16 operands, in an explicit order: the
// MFMAs of PV(t) (Oᵀ += Vᵀ P(t)) and then of Sᵀ(t+2) (accumulated onto `init`)
// alternate one by one with the weights of tile t+1 (P(t+1) = 2^(Sᵀ(t+1)·cs − m),
// rounded and packed in pairs, their fp32 values added to acc). A V or K register
// chunk is reloaded for two tiles ahead right after the last MFMA that reads it.
// sched_barrier pins the order: with one wavefront per SIMD, the MFMA pipe and
// the VALU only overlap where the instruction stream alternates, and the
// compiler's own schedule of this block leaves long runs of either kind.
// A wavefront-uniform address, marked as such so that a load from it plus a
// 32-bit lane offset takes the scalar-base form.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
using gbyte = const uint8_t __attribute__((address_space(1)));
using gu32x4 = const u32x4 __attribute__((address_space(1)));
__device__ __forceinline__ gbyte* sbase(const uint8_t* p) {
  const uint64_t b = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  return (gbyte*)(((uint64_t)hi << 32) | lo);
}

// One accumulator element into a VGPR, read where it is needed rather than as
// part of a copy of the whole accumulator. The unit of this file that is built
// with every MFMA result in VGPRs (PISA_FWD_VGPR_FORM: the bf16 fused pass and
// dense baseline) reads the value as it is, with no move.
__device__ __forceinline__ float acc_read(float x) {
#if PISA_FWD_VGPR_FORM
  return x;
#else
  float y;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(y) : "a"(x));
  return y;
#endif
}

template <int D, bool LAG, typename Wop>
__device__ __forceinline__ void xstep(typename Regs<bf16, D>::Acc& oacc,
                                      typename Regs<bf16, D>::V& vc,
                                      const typename Regs<bf16, D>::P& pc,
                                      typename Regs<bf16, D>::K& kc,
                                      const typename Regs<bf16, D>::Q& qr, f32x16 (&sx)[2],
                                      const f32x16& init, const f32x16 (&sy)[2],
                                      typename Regs<bf16, D>::P& py, float (&acc)[2],
                                      const Wop& wop, const uint8_t* vnext,
                                      const uint8_t* knext, int w, int lane) {
  using G = Geo<bf16, D>;
  typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
  constexpr int NV = G::DT * G::CPK;
  constexpr int NPV = 2 * NV, NM = NPV + 2 * G::NC;
  constexpr int EPM = 32 / NM;  // weights formed per MFMA
  static_assert(NM * EPM == 32, "32 weights per lane and sub-tile");
  uint32_t pw[2][4 * G::CPK];
  float xs[32], ps[32];
  // uniform base + 32-bit lane offset: the form global loads take with an SGPR
  // base, which issues faster than a 64-bit address per lane
  uint32_t lane_off = (uint32_t)lane * 16u;
  asm volatile("" : "+v"(lane_off));  // keeps base + lane offset from being hoisted as one 64-bit value
  // The addresses of this wavefront's part of the next V and K sub-tiles,
  // chunk x at x KiB, every load in the scalar-base form (uniform base plus a
  // 32-bit lane offset). Built with the accumulators in AGPRs (the per-block
  // first-order variant) one base per four chunks serves, the chunk offset
  // within them going to the load's immediate: 36 scalar instructions fewer per
  // 64 MFMAs, pb1 108.2-108.6 -> 103.9-104.0 ms. In the VGPR-form unit each
  // chunk keeps a base of its own: there the shared bases measured the fused
  // pass 1% slower (Wan 14.83-14.89 -> 15.00-15.03 ms), in one process.
#if PISA_FWD_VGPR_FORM
  auto vaddr = [&](int x) { return sbase(vnext + (size_t)((w * NV + x) * kWave * 16)); };
  auto kaddr = [&](int c) { return sbase(knext + (size_t)((w * G::NC + c) * kWave * 16)); };
#else
  gbyte* const vb[2] = {sbase(vnext + (size_t)(w * NV) * kWave * 16),
                        sbase(vnext + (size_t)(w * NV + 4) * kWave * 16)};
  gbyte* const kb[2] = {sbase(knext + (size_t)(w * G::NC) * kWave * 16),
                        sbase(knext + (size_t)(w * G::NC + 4) * kWave * 16)};
  auto vaddr = [&](int x) { return vb[x >> 2] + (x & 3) * kWave * 16; };
  auto kaddr = [&](int c) { return kb[c >> 2] + (c & 3) * kWave * 16; };
#endif
  sx[0] = init;
  sx[1] = init;
  // With LAG the weights run as a three-stage pipeline over the 32 elements, so
  // that no instruction reads a register the one before it wrote (each such
  // pair costs a wait state): in group g, element g's accumulator is read,
  // element g-1 is exponentiated, and the pair ending at element g-2 is rounded
  // and summed; two groups without an MFMA drain it. Without LAG each group
  // finishes its own element. Measured at the Wan shape, the lag speeds up the
  // dense sweep (every tile an L2 hit) by 3% and, with the present generation
  // wait, the sparse pass by 1.4-1.9% (Wan and Hunyuan, densities 0.125 and
  // 0.25), so every bf16 sweep uses it.
  constexpr int LG = LAG ? EPM : 0;
#pragma unroll
  for (int mi = 0; mi < NM + (LAG ? 2 : 0); ++mi) {
    if (mi < NPV) {
      const int x = mi >> 1, qt = mi & 1;
      Op<bf16>::mma(oacc[x / G::CPK][qt], vc[x], pc[qt][x % G::CPK]);
      if (qt == 1)
        vc[x] = __builtin_bit_cast(uint4, *(gu32x4*)(vaddr(x) + lane_off));
    } else if (mi < NM) {
      const int c = (mi - NPV) >> 1, qt = (mi - NPV) & 1;
      Op<bf16>::mma(sx[qt], kc[c], qr[qt][c]);
      if (qt == 1)
        kc[c] = __builtin_bit_cast(uint4, *(gu32x4*)(kaddr(c) + lane_off));
    }
#pragma unroll
    for (int u = 0; u < EPM; ++u) {
      const int ea = mi * EPM + u, eb = ea - LG, ec = ea - 2 * LG;
      if (ea < 32) xs[ea] = acc_read(sy[ea >> 4][ea & 15]);
      if (eb >= 0 && eb < 32) ps[eb] = wop(xs[eb], eb >> 4);
      if (ec >= 0 && ec < 32 && (ec & 1)) {
        const int qt = ec >> 4, r = ec & 15;
        const bf16x2 pr = {(bf16)ps[ec - 1], (bf16)ps[ec]};
        acc[qt] += ps[ec - 1] + ps[ec];
        pw[qt][r >> 1] = __builtin_bit_cast(uint32_t, pr);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int c = 0; c < G::CPK; ++c)
      py[qt][c] = make_uint4(pw[qt][4 * c], pw[qt][4 * c + 1], pw[qt][4 * c + 2], pw[qt][4 * c + 3]);
}

// Start values of the 16 Sᵀ accumulator elements of a lane from a bit mask of
// its keys (bit vkey(r, 0) set: key r takes no weight): −inf or 0. The bit,
// sign-extended and shifted into the exponent field, gives 0xFF800000 (−inf)
// or 0 in two integer operations, with no compare, no condition register, and
// none of the wait states a condition select needs before an MFMA reads it.
__device__ __forceinline__ f32x16 dead_init(uint32_t dh) {
  f32x16 v;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int s = (int)(dh << (31 - vkey(r, 0))) >> 31;  // 0 or -1
    v[r] = __builtin_bit_cast(float, (uint32_t)s << 23);
  }
  return v;
}

// Keys of a wavefront's 32 that lie past the end of the sequence, as a bit
// mask (bit k: key k), given how many of them are valid.
__device__ __forceinline__ uint32_t dead_keys(int nvalid) {
  return nvalid >= 32 ? 0u : (nvalid <= 0 ? ~0u : ~((1u << nvalid) - 1u));
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

// Software-pipelined loop over nt sub-tiles. off(t) gives tile t's byte offset
// from kbase / vbase and init(t) the accumulator start of its Sᵀ; init_loop(t)
// is the same for the tiles whose Sᵀ the main loop forms (t < nt - 2), where it
// may be a constant. The weights' row sums go to acc. Per tile t the MFMA pipe
// runs PV(t) then Sᵀ(t+2) while the VALU forms P(t+1) from Sᵀ(t+1). K and V are double-buffered in registers: the
// loads of V(t+2) and K(t+4) are issued during tile t, two tiles before use,
// which hides the latency of gathers that miss the L2. RSUM: see weights_full.
template <typename T, int D, bool LAG, bool RSUM, typename Off, typename InitL, typename Init>
__device__ __forceinline__ void pipelined(int nt, const uint8_t* kbase, const uint8_t* vbase,
                                          const Off& off, const InitL& init_loop, const Init& init,
                                          float (&acc)[2],
                                          const float (&m)[2], float cs,
                                          const typename Regs<T, D>::Q& qr,
                                          typename Regs<T, D>::Acc& oacc, int w, int lane) {
  if (nt <= 0) return;
  auto wts = [&](const f32x16 (&sx)[2], typename Regs<T, D>::P& px) {
    weights_full<T, D, RSUM>(sx, m, acc, px, cs);
  };
  auto wexp = [&](float x, int qt) { return __builtin_amdgcn_exp2f(fmaf(x, cs, -m[qt])); };
  typename Regs<T, D>::K kc0, kc1;
  typename Regs<T, D>::V vc0, vc1;
  f32x16 sa[2], sb[2];
  typename Regs<T, D>::P pa, pb;
  auto ldk = [&](typename Regs<T, D>::K& kc, int t) { load_k<T, D>(kbase + off(t), w, lane, kc); };
  auto ldv = [&](typename Regs<T, D>::V& vc, int t) { load_v<T, D>(vbase + off(t), w, lane, vc); };
  auto sm = [&](const typename Regs<T, D>::K& kc, f32x16 (&sx)[2], int t) {
    mma_s<T, D>(qr, kc, sx, init(t));
  };
  auto sm_loop = [&](const typename Regs<T, D>::K& kc, f32x16 (&sx)[2], int t) {
    mma_s<T, D>(qr, kc, sx, init_loop(t));
  };
  // The prologue has no conditions (tiles past the end are replaced by the
  // last one, and Sᵀ(1) of a one-tile run is never used), so that every path
  // into the loop has issued the same loads in the same order: the waits the
  // compiler places in the loop then only cover the tile about to be used.
  const int tl = nt - 1;
  ldk(kc0, 0);
  ldv(vc0, 0);
  ldk(kc1, min(1, tl));
  ldv(vc1, min(1, tl));
  sm(kc0, sa, 0);
  ldk(kc0, min(2, tl));
  wts(sa, pa);
  sm(kc1, sb, 1);
  ldk(kc1, min(3, tl));
  int t = 0;
  // invariant at the top: pa = P(t), sb = S(t+1), kc0 = K(t+2), kc1 = K(t+3),
  // vc0 = V(t), vc1 = V(t+1) (each where the tile exists)
  for (; t + 5 < nt; t += 2) {
    if constexpr (sizeof(T) == 2) {
      xstep<D, LAG>(oacc, vc0, pa, kc0, qr, sa, init_loop(t + 2), sb, pb, acc, wexp, vbase + off(t + 2),
               kbase + off(t + 4), w, lane);  // PV(t), S(t+2), P(t+1)
      xstep<D, LAG>(oacc, vc1, pb, kc1, qr, sb, init_loop(t + 3), sa, pa, acc, wexp, vbase + off(t + 3),
               kbase + off(t + 5), w, lane);  // PV(t+1), S(t+3), P(t+2)
    } else {
      mma_pv<T, D>(oacc, vc0, pa);  // PV(t)
      ldv(vc0, t + 2);
      sm_loop(kc0, sa, t + 2);      // S(t+2)
      ldk(kc0, t + 4);
      wts(sb, pb);                  // P(t+1)
      interleave_tile();
      mma_pv<T, D>(oacc, vc1, pb);  // PV(t+1)
      ldv(vc1, t + 3);
      sm_loop(kc1, sb, t + 3);      // S(t+3)
      ldk(kc1, t + 5);
      wts(sa, pa);                  // P(t+2)
      interleave_tile();
    }
  }
  // 1 to 5 tiles left
  const int r = nt - t;
  mma_pv<T, D>(oacc, vc0, pa);                                   // tile t
  if (r >= 2) {
    if (r >= 3) {
      ldv(vc0, t + 2);
      sm(kc0, sa, t + 2);
      if (r >= 5) ldk(kc0, t + 4);
    }
    wts(sb, pb);
    mma_pv<T, D>(oacc, vc1, pb);                                 // tile t+1
    if (r >= 3) {
      if (r >= 4) {
        ldv(vc1, t + 3);
        sm(kc1, sb, t + 3);
      }
      wts(sa, pa);
      mma_pv<T, D>(oacc, vc0, pa);                               // tile t+2
      if (r >= 4) {
        if (r >= 5) {
          ldv(vc0, t + 4);
          sm(kc0, sa, t + 4);
        }
        wts(sb, pb);
        mma_pv<T, D>(oacc, vc1, pb);                             // tile t+3
        if (r >= 5) {
          wts(sa, pa);
          mma_pv<T, D>(oacc, vc0, pa);                           // tile t+4
        }
      }
    }
  }
}

// Sums the two wavefronts' partial states (wavefront W finishes output tiles
// W*DH .. W*DH+DH-1), adds the first-order term and stores o = N / D (and, when
// a.lse is set, ln D_t for a backward pass). In the fast kernel a tile whose
// denominator is too small is queued for the careful kernel and nothing is
// stored.
template <typename T, int D, bool CAREFUL, int W>
__device__ __forceinline__ void epilogue(const FwdArgs& a, typename Regs<T, D>::Acc& oacc,
                                         float (&m)[2], float (&l)[2], float (&asum)[2],
                                         const typename Regs<T, D>::Q& qr, FwdShared<T, D>& sh,
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
    float mt = m[qt];
    if constexpr (CAREFUL) {
      const float mstar = fmaxf(m[qt], mp);
      fs = (m[qt] == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(m[qt] - mstar);
      fp = (mp == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(mp - mstar);
      mt = mstar;
    }
    Lt[qt] = fs * l[qt] + fp * lp;
    At[qt] = fs * asum[qt] + fp * ap;
    const int row = r0 + 32 * qt + l32;
    // ln D_t = (shift + log2 of the shifted sum) · ln 2, when asked for (a
    // tile the fast kernel hands to the careful kernel is written again there)
    if (a.lse != nullptr && w == 0 && h == 0 && row < a.L)
      a.lse[(size_t)bh * a.L + row] = (mt + __log2f(Lt[qt])) * kLn2;
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
        uint8_t* dst = io_row<true>(a, bh, row) + (size_t)d * ESZ;
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
template <typename T, int D, bool CAREFUL, int SPB, bool DENSE, typename Before, typename After>
__device__ __forceinline__ void query_tile(const FwdArgs& a, long item, FwdShared<T, D>& sh,
                                           typename Regs<T, D>::Xo& xo, const Before& before_exact,
                                           const After& after_exact) {
  using G = Geo<T, D>;
  constexpr int NC = G::NC, DT = G::DT, ESZ = G::ESZ, KW = G::KW;
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  constexpr int spb = SPB;
  const int half = (int)(item % spb);
  const long rest = item / spb;
  const int i = (int)(rest % a.n);
  const long bh = rest / a.n;
  const int r0 = i * a.blk + half * kSub;
  if (r0 >= a.L) {
    after_exact();
    return;
  }

  constexpr bool dense = DENSE;
  const int nsel = dense ? a.n : a.topk;
  // The selection is read-only during the launch. Reading it through the
  // constant address space makes its (uniform) loads scalar loads, which are
  // counted apart from the vector loads: taking the next block index never waits
  // for the K/V gathers already in flight.
  using cidx_t = const int32_t __attribute__((address_space(4)));
  const cidx_t* myidx = dense ? nullptr : (const cidx_t*)(a.idx + (bh * a.n + i) * (long)a.topk);
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
      qr[qt][c] = row < a.L ? *(const uint4*)(io_row<false>(a, bh, row) + (size_t)d0 * ESZ)
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
        qn2[qt] = Op<T>::dot(qr[qt][c], qr[qt][c], qn2[qt]);
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

  typename Regs<T, D>::K kc;  // careful kernel only
  typename Regs<T, D>::V vc;

  // ---- phase 2: zeroth-order terms of the unselected blocks
  auto phase2 = [&]() {
    if (tail) {
      const size_t head_ct = (size_t)bh * a.nct;
      const float blk_w = (float)a.blk, last_w = (float)(a.n_last - a.blk);
      if constexpr (!CAREFUL) {
        // selected and padding centroids start at −inf, so they get weight 0;
        // their row sums go to A_t, from which D gets n_j per centroid later
        auto cinit = [&](int ct) {
          const int jbase = kSub * ct + 32 * w;
          const int nvalid = a.n - jbase;  // valid centroids from this wavefront's first key
          const uint32_t dh = (sh.selmask[jbase >> 5] | dead_keys(nvalid)) >> (4 * h);
          const f32x16 v = dead_init(dh);
          return v;
        };
        pipelined<T, D, true, false>(
            a.nct, a.kbp, a.vbp, [&](int ct) -> size_t { return (head_ct + ct) * G::SUB_BYTES; },
            cinit, cinit, asum, m, cs, qr, oacc, w, lane);
      } else {
        load_k<T, D>(a.kbp + head_ct * G::SUB_BYTES, w, lane, kc);
        load_v<T, D>(a.vbp + head_ct * G::SUB_BYTES, w, lane, vc);
        for (int ct = 0; ct < a.nct; ++ct) {
          const bool more = ct + 1 < a.nct;
          const int jbase = kSub * ct + 32 * w;
          const uint32_t word = sh.selmask[jbase >> 5];
          const size_t nxt = (head_ct + ct + 1) * G::SUB_BYTES;
          step<T, D, true, kCentroid>(oacc, qr, kc, vc, m, l, asum, cs, h, w, lane, a.n - kSub * ct,
                                      word, a.n - 1 - jbase, blk_w, last_w,
                                      more ? a.kbp + nxt : nullptr, more ? a.vbp + nxt : nullptr);
        }
      }
    }
  };

  // ---- phase 1: exact selected blocks, ascending
  const size_t head_sub = (size_t)bh * a.n * spb;
  const int nsub_last = (a.n_last + kSub - 1) / kSub;
  if constexpr (!CAREFUL) {
    // With a fixed shift the order of the terms does not matter. For short
    // exact sweeps the centroid scan comes first: it reads only the k̄ / ΣV
    // tiles, which every query tile of the head shares, and fills the time a
    // workgroup would otherwise spend in before_exact (the generation wait that
    // lines up the exact sweeps over the gathered blocks). For long sweeps it
    // comes last, after the point where a workgroup with a short centroid scan
    // already counts as done for the generation wait; running it first there
    // measured slower at the Wan and Hunyuan shapes.
    const bool centroids_first = nsel * spb < kCentroidsFirstBelow;
    if (centroids_first) phase2();
    before_exact();
    // Full sub-tiles, software-pipelined two deep: Sᵀ of tile t+1 is issued
    // before the weights of tile t, so the MFMA pipe works while the VALU
    // exponentiates. The short last block (always last: indices ascend) is
    // left to the masked loop below.
    const bool ragged_last = a.n_last < a.blk && block_at(nsel - 1) == a.n - 1;
    // The short last block, if selected, is always last (indices ascend): its
    // sub-tiles close the same pipeline, with keys beyond n_last starting at
    // −inf. The main loop never forms Sᵀ of the last two sub-tiles, so its own
    // initial value stays the constant zero.
    const int nt_full = (nsel - (ragged_last ? 1 : 0)) * spb;
    const int nt = nt_full + (ragged_last ? nsub_last : 0);
    // (the short block is the selection's last entry, so the same formula
    // addresses its sub-tiles)
    auto off = [&](int t) -> size_t {
      return (head_sub + (size_t)block_at(t / spb) * spb + (t % spb)) * G::SUB_BYTES;
    };
    auto init = [&](int t) {
      const uint32_t dh =
          (t < nt_full ? 0u : dead_keys(a.n_last - kSub * (t - nt_full) - 32 * w)) >> (4 * h);
      const f32x16 v = dead_init(dh);
      return v;
    };
    pipelined<T, D, true, true>(
        nt, a.kp, a.vp, off, [](int) { return f32x16{}; }, init, l, m, cs, qr, oacc, w, lane);
    after_exact();
    if (!centroids_first) phase2();
  } else {
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
        step<T, D, true, kExactFull>(oacc, qr, kc, vc, m, l, asum, cs, h, w, lane, valid, 0u, -1,
                                     0.f, 0.f, kn, vn);
      else
        step<T, D, true, kExactRagged>(oacc, qr, kc, vc, m, l, asum, cs, h, w, lane, valid, 0u,
                                       -1, 0.f, 0.f, kn, vn);
      if (!more) break;
      s = s2;
      st = st2;
      j = j2;
    }
    phase2();
  }

  // fast kernel: D gets n_j per unselected block, i.e. blk·A_t, corrected for
  // the short last block by (n_last − blk)·α_t,n−1 (counted once: wavefront 0,
  // lane half 0)
  if constexpr (!CAREFUL) {
    if (tail) {
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) l[qt] = fmaf((float)a.blk, asum[qt], l[qt]);
      const int jl = a.n - 1;
      if (a.n_last != a.blk && !((sh.selmask[jl >> 5] >> (jl & 31)) & 1u)) {
        const int kk = jl & 63;
        const uint8_t* tile = a.kbp + ((size_t)bh * a.nct + (jl >> 6)) * G::SUB_BYTES;
        const int lx = h * 32 + (kk & 31);
        float dot[2] = {0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const uint4 kch = *(const uint4*)(tile + (((kk >> 5) * NC + c) * kWave + lx) * 16);
          dot[0] = Op<T>::dot(kch, qr[0][c], dot[0]);
          dot[1] = Op<T>::dot(kch, qr[1][c], dot[1]);
        }
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          const float d = dot[qt] + __shfl_xor(dot[qt], 32);
          const float alpha = __builtin_amdgcn_exp2f(fmaf(d, cs, -m[qt]));
          if (w == 0 && h == 0) l[qt] = fmaf((float)(a.n_last - a.blk), alpha, l[qt]);
        }
      }
    }
  }

  // ---- merge, first-order term, output (wave-uniform branch: every register
  // index is a compile-time constant)
  if (w == 0)
    epilogue<T, D, CAREFUL, 0>(a, oacc, m, l, asum, qr, sh, xo, tail, bh, r0, lane, item);
  else
    epilogue<T, D, CAREFUL, 1>(a, oacc, m, l, asum, qr, sh, xo, tail, bh, r0, lane, item);
}

// ---------------------------------------------------------------------------
// Per-block first-order variant. An unselected block j contributes
// α_tj (ΣV_j + s q_t H_j) to N_t, which expands over the block's own keys as
// Σ_n α_tj (1 + s q_t·(k_n − k̄_j)) v_n: the first-order Taylor expansion of
// e^{ℓ_tn} about the centroid logit. So the variant visits every key block:
// the selected ones with exponential weights (the hybrid's exact sweep), the
// unselected ones with linear weights P = α_tj (1 + ℓ_tn − c_tj), on the same
// MFMA operand copies of K and V; no D×D matrix per block is stored or read.
// The centroid logits c_tj come from the k̄ tiles, 64 blocks at a time,
// through LDS.

// Linear weights of one sub-tile of an unselected block: P = a1·Sᵀ + b1 per
// query row (a1 = α s, b1 = α (1 − s C)), and their row sums. RAGGED: keys past
// the end of the sequence carry −inf in Sᵀ and get weight 0.
template <typename T, int D, bool RAGGED>
__device__ __forceinline__ void weights_linear(const f32x16 (&sacc)[2], const float (&a1)[2],
                                               const float (&b1)[2], float (&l)[2],
                                               typename Regs<T, D>::P& pc) {
  using G = Geo<T, D>;
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
#pragma unroll
    for (int c = 0; c < G::CPK; ++c) {
      float p[G::KW];
#pragma unroll
      for (int e = 0; e < G::KW; ++e) {
        const float sv = acc_read(sacc[qt][G::KW * c + e]);  // one at a time: few live VGPRs
        const float x = fmaf(sv, a1[qt], b1[qt]);
        p[e] = (RAGGED && sv == kNegInf) ? 0.0f : x;
      }
      pc[qt][c] = Op<T>::pack(p);
      Op<T>::unpack(pc[qt][c], p);  // the sums take the rounded weights
#pragma unroll
      for (int e = 0; e < G::KW; e += 2) l[qt] += p[e] + p[e + 1];
    }
  }
}

// Software-pipelined sweep over nt sub-tiles with per-tile weights (same
// schedule as `pipelined`: PV(t) and Sᵀ(t+2) on the MFMA pipe while the VALU
// forms P(t+1); K and V double-buffered two tiles ahead; loads past the end
// clamped to the last tile). wts(Sᵀ, P, t) forms tile t's weights in the
// prologue and the last tiles; in the main loop, which never reaches the last
// two tiles, bf16 takes the written-out xstep with the linear weights
// P = fma(Sᵀ, A, B) of coef(t, A, B), and row sums into acc.
template <typename T, int D, typename Off, typename Init, typename Wts, typename Coef>
__device__ __forceinline__ void pipelined_w(int nt, const uint8_t* kbase, const uint8_t* vbase,
                                            const Off& off, const Init& init, const Wts& wts,
                                            const Coef& coef, float (&acc)[2],
                                            const typename Regs<T, D>::Q& qr,
                                            typename Regs<T, D>::Acc& oacc, int w, int lane) {
  if (nt <= 0) return;
  typename Regs<T, D>::K kc0, kc1;
  typename Regs<T, D>::V vc0, vc1;
  f32x16 sa[2], sb[2];
  typename Regs<T, D>::P pa, pb;
  auto ldk = [&](typename Regs<T, D>::K& kc, int t) { load_k<T, D>(kbase + off(t), w, lane, kc); };
  auto ldv = [&](typename Regs<T, D>::V& vc, int t) { load_v<T, D>(vbase + off(t), w, lane, vc); };
  auto sm = [&](const typename Regs<T, D>::K& kc, f32x16 (&sx)[2], int t) {
    mma_s<T, D>(qr, kc, sx, init(t));
  };
  const int tl = nt - 1;
  ldk(kc0, 0);
  ldv(vc0, 0);
  ldk(kc1, min(1, tl));
  ldv(vc1, min(1, tl));
  sm(kc0, sa, 0);
  ldk(kc0, min(2, tl));
  wts(sa, pa, 0);
  sm(kc1, sb, min(1, tl));
  ldk(kc1, min(3, tl));
  int t = 0;
  // top of the loop: pa = P(t), sb = Sᵀ(t+1), kc0 = K(t+2), kc1 = K(t+3),
  // vc0 = V(t), vc1 = V(t+1)
  for (; t + 5 < nt; t += 2) {
    if constexpr (sizeof(T) == 2) {
      float A1[2], B1[2], A2[2], B2[2];
      coef(t + 1, A1, B1);
      coef(t + 2, A2, B2);
      auto w1 = [&](float x, int qt) { return fmaf(x, A1[qt], B1[qt]); };
      auto w2 = [&](float x, int qt) { return fmaf(x, A2[qt], B2[qt]); };
      xstep<D, true>(oacc, vc0, pa, kc0, qr, sa, f32x16{}, sb, pb, acc, w1, vbase + off(t + 2),
                     kbase + off(t + 4), w, lane);  // PV(t), Sᵀ(t+2), P(t+1)
      xstep<D, true>(oacc, vc1, pb, kc1, qr, sb, f32x16{}, sa, pa, acc, w2, vbase + off(t + 3),
                     kbase + off(t + 5), w, lane);  // PV(t+1), Sᵀ(t+3), P(t+2)
    } else {
      mma_pv<T, D>(oacc, vc0, pa);
      ldv(vc0, t + 2);
      sm(kc0, sa, t + 2);
      ldk(kc0, t + 4);
      wts(sb, pb, t + 1);
      interleave_tile();
      mma_pv<T, D>(oacc, vc1, pb);
      ldv(vc1, t + 3);
      sm(kc1, sb, t + 3);
      ldk(kc1, t + 5);
      wts(sa, pa, t + 2);
      interleave_tile();
    }
  }
  const int r = nt - t;  // 1 to 5 tiles left
  mma_pv<T, D>(oacc, vc0, pa);
  if (r >= 2) {
    if (r >= 3) {
      ldv(vc0, t + 2);
      sm(kc0, sa, t + 2);
      if (r >= 5) ldk(kc0, t + 4);
    }
    wts(sb, pb, t + 1);
    mma_pv<T, D>(oacc, vc1, pb);
    if (r >= 3) {
      if (r >= 4) {
        ldv(vc1, t + 3);
        sm(kc1, sb, t + 3);
      }
      wts(sa, pa, t + 2);
      mma_pv<T, D>(oacc, vc0, pa);
      if (r >= 4) {
        if (r >= 5) {
          ldv(vc0, t + 4);
          sm(kc0, sa, t + 4);
        }
        wts(sb, pb, t + 3);
        mma_pv<T, D>(oacc, vc1, pb);
        if (r >= 5) {
          wts(sa, pa, t + 4);
          mma_pv<T, D>(oacc, vc0, pa);
        }
      }
    }
  }
}

// The per-block first-order pass of one 64-row query tile. The selected blocks
// take the hybrid's exponential sweep; then, 64 blocks at a time, the centroid
// logits go to `cl` (a 64 x 64 LDS array, raw q·k̄, [block][query row]), the
// group's unselected blocks are listed in `ul` (64 LDS entries), and a sweep
// with linear weights only runs over them. The fast
// kernel shifts every exponent by the Cauchy–Schwarz bound of the logits, as
// the hybrid's fast kernel does; the careful kernel (a tile whose denominator
// underflowed) first finds the largest exponent the tile actually uses: the
// exact logits of its selected blocks and the centroid logits of the others.
template <typename T, int D, bool CAREFUL, int SPB, typename Before, typename After>
__device__ __forceinline__ void pb1_tile(const FwdArgs& a, long item, FwdShared<T, D>& sh,
                                         typename Regs<T, D>::Xo& xo, float (*cl)[kSub], int* ul,
                                         const Before& before_sweep, const After& after_sweep) {
  using G = Geo<T, D>;
  constexpr int NC = G::NC, DT = G::DT, ESZ = G::ESZ, KW = G::KW;
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr int spb = SPB;
  const int half = (int)(item % spb);
  const long rest = item / spb;
  const int i = (int)(rest % a.n);
  const long bh = rest / a.n;
  const int r0 = i * a.blk + half * kSub;
  if (r0 >= a.L) {
    after_sweep();
    return;
  }
  const int nsel = a.topk;
  const int32_t* myidx = a.idx + (bh * a.n + i) * (long)a.topk;
  auto block_at = [&](int s) { return min(max(myidx[s], 0), a.n - 1); };
  {
    const int nw = (a.n + 31) >> 5;
    for (int x = tid; x < nw; x += 128) sh.selmask[x] = 0u;
    __syncthreads();
    for (int s = tid; s < nsel; s += 128) {
      const int j = block_at(s);
      atomicOr(&sh.selmask[j >> 5], 1u << (j & 31));
    }
    __syncthreads();
  }
  auto selected = [&](int j) { return ((sh.selmask[j >> 5] >> (j & 31)) & 1u) != 0u; };

  typename Regs<T, D>::Q qr;
  typename Regs<T, D>::Acc oacc;
  float m[2], l[2] = {0.f, 0.f}, asum[2] = {0.f, 0.f};
  const float cs = a.cs;
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int row = r0 + 32 * qt + l32;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int d0 = 2 * KW * c + KW * h;
      qr[qt][c] = row < a.L ? *(const uint4*)(io_row<false>(a, bh, row) + (size_t)d0 * ESZ)
                            : make_uint4(0, 0, 0, 0);
    }
  }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt][0] = oacc[dt][1] = f32x16{};

  const size_t head_sub = (size_t)bh * a.n * spb;
  const size_t head_ct = (size_t)bh * a.nct;
  const bool ragged = a.n_last < a.blk;
  const int nsub_last = (a.n_last + kSub - 1) / kSub;
  const int g_last = (a.n - 1) * spb;  // first sub-tile of the last block
  // Sᵀ start for global sub-tile g: −inf at keys past the end of the sequence
  auto init_g = [&](int g) {
    f32x16 v = f32x16{};
    if (ragged && g >= g_last) {
      const uint32_t dh = dead_keys(a.n_last - kSub * (g - g_last) - 32 * w) >> (4 * h);
      v = dead_init(dh);
    }
    return v;
  };

  if constexpr (!CAREFUL) {
    float qn2[2] = {0.f, 0.f};
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
      for (int c = 0; c < NC; ++c) qn2[qt] = Op<T>::dot(qr[qt][c], qr[qt][c], qn2[qt]);
    float km = 0.f;
    for (int c = lane; c < a.nch; c += kWave) km = fmaxf(km, a.kmax2[bh * a.nch + c]);
    km = wave_max(km);
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const float q2 = qn2[qt] + __shfl_xor(qn2[qt], 32);
      m[qt] = cs * sqrtf(q2 * km) - kHeadroom;
    }
  } else {
    float mx[2] = {kNegInf, kNegInf};
    typename Regs<T, D>::K kc;
    f32x16 sx[2];
    for (int s = 0; s < nsel; ++s) {
      const int j = block_at(s);
      const int nsub = (ragged && j == a.n - 1) ? nsub_last : spb;
      for (int st = 0; st < nsub; ++st) {
        const int g = j * spb + st;
        load_k<T, D>(a.kp + (head_sub + g) * G::SUB_BYTES, w, lane, kc);
        mma_s<T, D>(qr, kc, sx, init_g(g));
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx[qt] = fmaxf(mx[qt], sx[qt][r]);
      }
    }
    for (int ct = 0; ct < a.nct; ++ct) {
      load_k<T, D>(a.kbp + (head_ct + ct) * G::SUB_BYTES, w, lane, kc);
      mma_s<T, D>(qr, kc, sx);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = kSub * ct + 32 * w + vkey(r, h);
        if (j < a.n && !selected(j)) {
          mx[0] = fmaxf(mx[0], sx[0][r]);
          mx[1] = fmaxf(mx[1], sx[1][r]);
        }
      }
    }
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      mx[qt] = fmaxf(mx[qt], __shfl_xor(mx[qt], 32));
      if (h == 0) sh.xstat[w][0][qt][l32] = mx[qt];
    }
    __syncthreads();
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) m[qt] = fmaxf(mx[qt], sh.xstat[1 - w][0][qt][l32]) * cs;
    __syncthreads();
  }

  before_sweep();
  {
    // selected blocks: the hybrid's exact sweep (the short last block, if
    // selected, is the selection's last entry and closes the same pipeline)
    const bool ragged_last = ragged && block_at(nsel - 1) == a.n - 1;
    const int nt_full = (nsel - (ragged_last ? 1 : 0)) * spb;
    const int nt = nt_full + (ragged_last ? nsub_last : 0);
    auto off = [&](int t) -> size_t {
      return (head_sub + (size_t)block_at(t / spb) * spb + (t % spb)) * G::SUB_BYTES;
    };
    auto init = [&](int t) {
      const uint32_t dh =
          (t < nt_full ? 0u : dead_keys(a.n_last - kSub * (t - nt_full) - 32 * w)) >> (4 * h);
      const f32x16 v = dead_init(dh);
      return v;
    };
    pipelined<T, D, true, true>(nt, a.kp, a.vp, off, [](int) { return f32x16{}; }, init, l, m, cs, qr,
                          oacc, w, lane);
  }
  for (int ct = 0; ct < a.nct; ++ct) {
    const int j0 = kSub * ct, j1 = min(j0 + kSub, a.n);
    {
      typename Regs<T, D>::K kc;
      f32x16 sx[2];
      load_k<T, D>(a.kbp + (head_ct + ct) * G::SUB_BYTES, w, lane, kc);
      mma_s<T, D>(qr, kc, sx);
      // one base address per lane, the rest constant offsets
      float* clb = &cl[32 * w + 4 * h][l32];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int r = 0; r < 16; ++r) clb[(vkey(r, 0)) * kSub + 32 * qt] = sx[qt][r];
    }
    // the group's unselected blocks, ascending (both wavefronts count them;
    // wavefront 0 writes the list)
    const bool un = j0 + lane < j1 && !selected(j0 + lane);
    const uint64_t ub = __ballot(un);
    if (w == 0 && un) ul[__popcll(ub & ((1ull << lane) - 1ull))] = j0 + lane;
    const int nu = __popcll(ub);
    __syncthreads();
    // the short last block, if unselected, is the list's last entry
    const bool ragged_u = ragged && j1 == a.n && nu > 0 && !selected(a.n - 1);
    const int nt = nu * spb - (ragged_u ? spb - nsub_last : 0);
    auto gsub = [&](int t) { return ul[t / spb] * spb + t % spb; };
    auto off = [&](int t) -> size_t { return (head_sub + gsub(t)) * G::SUB_BYTES; };
    auto init = [&](int t) { return init_g(gsub(t)); };
    auto coef = [&](int t, float (&A)[2], float (&B)[2]) {
      const int j = ul[t / spb];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        const float c = cl[j - j0][32 * qt + l32];
        const float al = __builtin_amdgcn_exp2f(fmaf(c, cs, -m[qt]));
        A[qt] = al * a.scale;
        B[qt] = fmaf(-A[qt], c, al);
      }
    };
    auto wts = [&](const f32x16 (&sx)[2], typename Regs<T, D>::P& px, int t) {
      float a1[2], b1[2];
      coef(t, a1, b1);
      if (ragged && gsub(t) >= g_last)
        weights_linear<T, D, true>(sx, a1, b1, l, px);
      else
        weights_linear<T, D, false>(sx, a1, b1, l, px);
    };
    // (tiles of the main loop are never the ragged last ones)
    pipelined_w<T, D>(nt, a.kp, a.vp, off, init, wts, coef, l, qr, oacc, w, lane);
    __syncthreads();  // every wavefront is done with this group's logits and list
  }
  after_sweep();

  if (w == 0)
    epilogue<T, D, CAREFUL, 0>(a, oacc, m, l, asum, qr, sh, xo, false, bh, r0, lane, item);
  else
    epilogue<T, D, CAREFUL, 1>(a, oacc, m, l, asum, qr, sh, xo, false, bh, r0, lane, item);
}

}  // namespace

// The query tile of workgroup `wg` in generation g. Workgroups reach the chip's
// eight XCDs in turn (workgroup w to XCD w mod 8), and each XCD has its own L2.
// Within every full generation the workgroups of one XCD therefore take
// consecutive query tiles, not every eighth one: neighbouring query blocks
// share many of their selected key blocks (real selections are largely local)
// and all of their centroid tiles, so one L2 serves each gathered tile to
// more of the workgroups that need it. Measured at the Wan shape: fused pass
// 16.6 -> 15.1 ms with content-based selections, 25.7 -> 14.9 ms with a banded
// selection. The last, partial generation keeps the plain order.
__device__ __forceinline__ long tile_of(const FwdArgs& a, long wg, long g) {
  if ((g + 1) * a.nwg > a.total || (a.nwg & 7) != 0) return wg;
  const long r = wg - g * a.nwg;
  return g * a.nwg + (r & 7) * (a.nwg >> 3) + (r >> 3);
}

// One workgroup per query tile, in generations (tile_of maps workgroups to
// tiles): the workgroups of one XCD work on neighbouring query tiles of one head. Workgroups are grouped in generations
// of nwg (as many as can be resident: two per CU); before its exact sweep a
// workgroup of generation g waits until every workgroup of generation g-1 is
// done with its exact sweep. Since workgroups are dispatched in index order,
// those are all running or done by then; the wait keeps the resident
// workgroups' ascending sweeps over the key blocks in step, so one XCD's L2
// serves each gathered K/V tile to many of them. Measured with content-based
// selections at the Wan shape: 27.5 -> 17.1 ms; waiting for all of the previous
// generation rather than 90% of it took Hunyuan from 24.8 to 21.6 ms.
//
// "Done" is counted in one of two places. Where the centroid scan is short
// (at most kEarlySignalMaxCt tiles), wavefront 0 counts its workgroup right
// after the exact sweep, so the next generation's sweeps overlap this one's
// centroid scans: 17.1 -> 16.7 ms at Wan. Those next-generation workgroups
// whose slot is still held by a centroid scan start late, though, and the lag
// grows with the scan: with 30 or more centroid tiles (Hunyuan, or Wan at twice
// its length) the sweeps drift apart and the pass gets 1-4% slower, so there a
// workgroup counts only once it has finished. The wait only shapes timing: it
// is bounded by sync_ticks, and no result depends on it.
template <typename T, int D, int SPB, bool DENSE>
__global__ __launch_bounds__(128, 1) void k_pisa_fwd(FwdArgs a) {
  __shared__ FwdShared<T, D> sh;
  __shared__ typename Regs<T, D>::Xo xo;
  const long g = (long)blockIdx.x / a.nwg;
  const long item = tile_of(a, blockIdx.x, g);
  // Where a workgroup counts only once it has finished (long centroid
  // scans), there is one arrival counter per XCD: workgroup r of a
  // generation runs on XCD r mod 8, and the L2 whose reuse the wait serves is
  // that XCD's alone, so a workgroup waits only for its XCD's share of the
  // previous generation. Measured in one process on one box: Hunyuan
  // 19.59 -> 18.7-18.9 ms. With the early count (Wan) the chip-wide counter
  // stays: per XCD it measured 14.51-14.57 -> 14.74-14.77 ms.
  const bool early = a.nct <= kEarlySignalMaxCt;
  const bool per_xcd = !early && (a.nwg & 7) == 0;
  int* const cnt = a.sync + (per_xcd ? (int)((blockIdx.x - g * a.nwg) & 7) : 0);
  const int target = (int)(per_xcd ? g * (a.nwg >> 3) : g * a.nwg);
  auto wait = [&]() {
    if (g > 0) {
      if (threadIdx.x == 0) {
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        while (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target &&
               __builtin_amdgcn_s_memrealtime() - t0 < (uint64_t)a.sync_ticks)
          __builtin_amdgcn_s_sleep(2);
      }
      __syncthreads();
    }
  };
  auto done = [&]() {
    if (threadIdx.x == 0) __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  query_tile<T, D, false, SPB, DENSE>(a, item, sh, xo, wait, [&] {
    if (early) done();
  });
  if (!early) {
    __syncthreads();
    done();
  }
}

// Recomputes, with a running maximum, the query tiles the fast kernel queued.
template <typename T, int D, int SPB, bool DENSE>
__global__ __launch_bounds__(128, 1) void k_pisa_fwd_careful(FwdArgs a) {
  __shared__ FwdShared<T, D> sh;
  __shared__ typename Regs<T, D>::Xo xo;
  const int count = *(volatile int*)a.redo;
  for (int e = blockIdx.x; e < count; e += gridDim.x) {
    const long item = a.redo[1 + e];
    __syncthreads();  // shared state of the previous tile fully consumed
    query_tile<T, D, true, SPB, DENSE>(a, item, sh, xo, [] {}, [] {});
  }
}

// Per-block first-order variant: one workgroup per query tile, in the same
// generations as k_pisa_fwd (every tile sweeps all key blocks in ascending
// order, so lining the sweeps up lets one XCD's L2 serve each K/V tile to many
// of them).
template <typename T, int D, int SPB>
__global__ __launch_bounds__(128, 1) void k_pisa_pb1(FwdArgs a) {
  __shared__ FwdShared<T, D> sh;
  __shared__ typename Regs<T, D>::Xo xo;
  __shared__ float cl[kSub][kSub];
  __shared__ int ul[kSub];
  const long g = (long)blockIdx.x / a.nwg;
  const long item = tile_of(a, blockIdx.x, g);
  auto wait = [&]() {
    if (g > 0) {
      if (threadIdx.x == 0) {
        const int target = (int)(g * a.nwg);
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        while (__hip_atomic_load(a.sync, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target &&
               __builtin_amdgcn_s_memrealtime() - t0 < (uint64_t)a.sync_ticks)
          __builtin_amdgcn_s_sleep(2);
      }
      __syncthreads();
    }
  };
  auto done = [&]() {
    if (threadIdx.x == 0) __hip_atomic_fetch_add(a.sync, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  pb1_tile<T, D, false, SPB>(a, item, sh, xo, cl, ul, wait, done);
}

// The query tiles whose denominator underflowed under the fast kernel's shift,
// again with the largest exponent each tile uses as its shift.
template <typename T, int D, int SPB>
__global__ __launch_bounds__(128, 1) void k_pisa_pb1_careful(FwdArgs a) {
  __shared__ FwdShared<T, D> sh;
  __shared__ typename Regs<T, D>::Xo xo;
  __shared__ float cl[kSub][kSub];
  __shared__ int ul[kSub];
  const int count = *(volatile int*)a.redo;
  for (int e = blockIdx.x; e < count; e += gridDim.x) {
    const long item = a.redo[1 + e];
    __syncthreads();
    pb1_tile<T, D, true, SPB>(a, item, sh, xo, cl, ul, [] {}, [] {});
  }
}

namespace {
__global__ void k_zero_counters(int* redo, int* sync) {
  *redo = 0;
#pragma unroll
  for (int x = 0; x < kSyncCounters; ++x) sync[x] = 0;
}
}  // namespace

template <typename T, int D, int SPB, bool DENSE>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_zero_counters, dim3(1), dim3(1), 0, s, a.redo, a.sync);
  hipLaunchKernelGGL((k_pisa_fwd<T, D, SPB, DENSE>), dim3((unsigned)a.total), dim3(128), 0, s, a);
  hipLaunchKernelGGL((k_pisa_fwd_careful<T, D, SPB, DENSE>), dim3(256), dim3(128), 0, s, a);
  return hipGetLastError();
}

template <typename T, int D, int SPB>
static hipError_t launch_pb1_t(const FwdArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_zero_counters, dim3(1), dim3(1), 0, s, a.redo, a.sync);
  hipLaunchKernelGGL((k_pisa_pb1<T, D, SPB>), dim3((unsigned)a.total), dim3(128), 0, s, a);
  hipLaunchKernelGGL((k_pisa_pb1_careful<T, D, SPB>), dim3(256), dim3(128), 0, s, a);
  return hipGetLastError();
}

// Generations of resident workgroups: two 2-wave workgroups per CU.
static hipError_t set_generation(FwdArgs& a) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  a.nwg = 2L * cus < a.total ? 2L * cus : a.total;
  return hipSuccess;
}

#if PISA_FWD_VGPR_FORM
// This unit of the file holds the bf16 fused pass and dense baseline only. It
// is built with every MFMA result and accumulator in VGPRs, so the weights read
// the Sᵀ accumulators directly; the unit built the usual way holds the rest.
// Measured at the Wan shape on one box, same process: fused pass 15.37-15.43
// -> 15.08 ms, dense baseline 95.0 -> 92.4 ms, same output bits.
template <int D>
static hipError_t launch_fused_bf16(FwdArgs a, hipStream_t s) {
  hipError_t e = set_generation(a);
  if (e != hipSuccess) return e;
  const bool dense = a.idx == nullptr;
  if (a.blk == 64)
    return dense ? launch_fwd_t<bf16, D, 1, true>(a, s) : launch_fwd_t<bf16, D, 1, false>(a, s);
  return dense ? launch_fwd_t<bf16, D, 2, true>(a, s) : launch_fwd_t<bf16, D, 2, false>(a, s);
}

hipError_t launch_fwd_bf16(int D, const FwdArgs& a, hipStream_t s) {
  return D == 64 ? launch_fused_bf16<64>(a, s) : launch_fused_bf16<128>(a, s);
}
#else
template <typename T, int D>
static hipError_t launch_fwd_b(FwdArgs a, hipStream_t s) {
  hipError_t e = set_generation(a);
  if (e != hipSuccess) return e;
  const bool dense = a.idx == nullptr;
  if (a.per_block && !dense)
    return a.blk == 64 ? launch_pb1_t<T, D, 1>(a, s) : launch_pb1_t<T, D, 2>(a, s);
  if constexpr (sizeof(T) == 2) {
    return launch_fwd_bf16(D, a, s);
  } else {
    if (a.blk == 64)
      return dense ? launch_fwd_t<T, D, 1, true>(a, s) : launch_fwd_t<T, D, 1, false>(a, s);
    return dense ? launch_fwd_t<T, D, 2, true>(a, s) : launch_fwd_t<T, D, 2, false>(a, s);
  }
}

hipError_t launch_fwd(int dtype, int D, const FwdArgs& a, hipStream_t s) {
  if (dtype == 1) return D == 64 ? launch_fwd_b<bf16, 64>(a, s) : launch_fwd_b<bf16, 128>(a, s);
  return D == 64 ? launch_fwd_b<float, 64>(a, s) : launch_fwd_b<float, 128>(a, s);
}
#endif

}  // namespace pisa
