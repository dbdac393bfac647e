// Joint backward of the attention-KL primitive for gfx950: the gradients of
// both settings -- (Q1, K1) for "optimise P1" and (Q2, K2) for "optimise P2"
// -- from one recompute of the two logit tiles and one pair of exponentials
// per (query, key) pair.
//
// Both settings rebuild P_k = 2^(t_k - LSE_k log2 e) tile by tile from the
// saved LSEs (agidaily.cc StreamKL article, section "Backward:
// recompute-based tile-by-tile gradients") and share every step up to dS:
//   dS2 = g (P2 - P1)                    (student, P1 fixed)
//   dS1 = g P1 (ln2 (u1 - u2) - KL)      (teacher, P2 fixed; u_k = t_k - L_k)
// so one kernel pass per side of the contraction produces all four
// gradients: the joint dK kernel owns keys (dK1 += dS1ᵀ Q1, dK2 += dS2ᵀ Q2),
// the joint dQ kernel owns queries (dQ1 += dS1 K1, dQ2 += dS2 K2).  Against
// the two settings run one after the other this saves one logit recompute
// and one exponential per pair in each kernel.
//
// The two sets of gradient accumulators (128 fp32 registers per lane at
// d = 128) do not fit two waves per SIMD, so these kernels run one wave per
// SIMD with the accumulators in the accumulation registers.  With no second
// wave to hide latency, each wave hides its own: every operand fragment of
// a block is read before its MFMA chains, the gradient operands before the
// dS work, and the mask-free steps run their two 32-row (32-key) blocks as a
// software pipeline (block 1's reads issued right after block 0's MFMA
// chains, so they land during block 0's dS work).  Doing about two thirds of
// the instructions of the two settings run one after the other, the kernels
// also run at a higher clock under the chip's power limit, and the joint
// call takes about 0.8x the time of the two split calls.  The tile layout,
// operand orders and masking follow bwd_split.hip.

#include <type_traits>

#include "skl_device.h"
#include "skl_internal.h"

namespace skl {

namespace {

// |g| goes into the exponents: with k = log2 |g| and the row constants
// A_k = LSE_k log2 e - k, w_k = t_k - A_k gives 2^w_k = |g| P_k, and
//   sign(g) dS2 = 2^w2 - 2^w1,   sign(g) dS1 = 2^w1 (ln2 (w1 - w2) - KL)
// (k cancels in w1 - w2).  Six vector ops and two exponentials per element;
// the sign of g multiplies the finished dQ rows, and dS only in the rare dK
// tiles that have a row with g < 0.  A row with g = 0 gets A1 = A2 = kZeroRow:
// both exponentials are 0 and w1 - w2 = 0, so both dS are exactly 0.
constexpr float kZeroRow = 1e30f;

__device__ __forceinline__ void joint_row_consts(float lse1, float lse2, float g, float& A1, float& A2) {
  if (g == 0.f) {
    A1 = kZeroRow;
    A2 = kZeroRow;
    return;
  }
  const float k = log2f(fabsf(g));
  A1 = fmaf(lse1, kLog2e, -k);
  A2 = fmaf(lse2, kLog2e, -k);
}

__device__ __forceinline__ void dS_both_abs(float s1, float s2, float c1, float c2, float A1, float A2, float kl,
                                            float& ds1, float& ds2) {
  const float w1 = fmaf(s1, c1, -A1);
  const float w2 = fmaf(s2, c2, -A2);
  const float e1 = exp2_hw(w1), e2 = exp2_hw(w2);
  ds2 = e2 - e1;
  ds1 = e1 * fmaf(w1 - w2, kLn2, -kl);
}

}  // namespace

// ---------------------------------------------------------------------------
// Joint dK kernel: 4 waves own 128 keys (32 each) of one (b, h) and walk the
// query tiles of 64 rows that see them, 32 rows at a time.  K fragments of
// both sides stay in registers; Q1/Q2 tiles come straight into a
// double-buffered swizzled LDS ring with the row constants (A1, A2, KL and
// the sign of g) beside them.
// ---------------------------------------------------------------------------
template <typename T, int D1, int D2, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void bwd_joint_dk_kernel(const BwdParams p) {
  using M = Mfma<T>;
  using frag = typename M::frag;
  constexpr int KC = M::KC, EPL = M::EPL;
  constexpr int NC1 = D1 / KC, NC2 = D2 / KC;
  constexpr int NB1 = D1 / 32, NB2 = D2 / 32;  // 32-wide column blocks of dK1 / dK2
  constexpr int ESZ = sizeof(T);
  constexpr int BQ = kDkBQ;
  constexpr int RB1 = D1 * ESZ, RB2 = D2 * ESZ;  // bytes per query row
  using T1 = SwzTile<RB1>;
  using T2 = SwzTile<RB2>;

  // Ring stages as separate LDS variables, so that the compiler can tell
  // reads of one stage from the direct-to-LDS loads in flight into the other.
  __shared__ __attribute__((aligned(1024))) char sQ1a[BQ * RB1], sQ1b[BQ * RB1];
  __shared__ __attribute__((aligned(1024))) char sQ2a[BQ * RB2], sQ2b[BQ * RB2];
  // Per query row of a tile: A1, A2, KL and sign(g); plus a flag per stage:
  // some row of the tile has g < 0.
  __shared__ __attribute__((aligned(16))) float sVa[4][BQ], sVb[4][BQ];
  __shared__ int sNeg[2];

  auto sQ1 = [&](int st) __attribute__((always_inline)) -> char* { return st ? sQ1b : sQ1a; };
  auto sQ2 = [&](int st) __attribute__((always_inline)) -> char* { return st ? sQ2b : sQ2a; };
  auto sVec = [&](int st) __attribute__((always_inline)) -> float(*)[BQ] { return st ? sVb : sVa; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int half = lane >> 5, col = lane & 31;

  const int64_t t = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t bh = t / p.num_ktiles;
  const int kt = (int)(t % p.num_ktiles);
  const int64_t b = bh / p.H, h = bh % p.H;
  const int64_t off = p.NK - p.NQ;
  const int64_t kt0 = (int64_t)kt * kBwdBK;
  const int64_t kw0 = kt0 + 32 * wave;
  const int64_t key = kw0 + col;
  const bool kvalid = key < p.NK;

  const char* const q1p = (const char*)p.q1 + (b * p.sq1.b + h * p.sq1.h) * ESZ;
  const char* const q2p = (const char*)p.q2 + (b * p.sq2.b + h * p.sq2.h) * ESZ;
  const char* const k1p = (const char*)p.k1 + (b * p.sk1.b + h * p.sk1.h) * ESZ;
  const char* const k2p = (const char*)p.k2 + (b * p.sk2.b + h * p.sk2.h) * ESZ;

  frag kf1[NC1], kf2[NC2];
#pragma unroll
  for (int c = 0; c < NC1; ++c)
    kf1[c] = kvalid ? M::load(k1p + (key * p.sk1.n + c * KC + half * EPL) * ESZ) : M::zero();
#pragma unroll
  for (int c = 0; c < NC2; ++c)
    kf2[c] = kvalid ? M::load(k2p + (key * p.sk2.n + c * KC + half * EPL) * ESZ) : M::zero();

  f32x16 dk1[NB1], dk2[NB2];
#pragma unroll
  for (int cb = 0; cb < NB1; ++cb) dk1[cb] = f32x16{};
#pragma unroll
  for (int cb = 0; cb < NB2; ++cb) dk2[cb] = f32x16{};

  int64_t qbeg = 0;
  if (CAUSAL) qbeg = max((int64_t)0, kt0 - off) / BQ * BQ;
  const int64_t nsteps = (p.NQ - qbeg + BQ - 1) / BQ;

  // Row values of the next query tile (LSE1, LSE2, g, KL) are loaded by the
  // first wave, one row per lane; the fetch only loads them and the stash,
  // after the step's compute, forms the row constants, so no wave waits for
  // the next tile's loads mid-step (any arithmetic on a loaded value makes it
  // wait for all of its outstanding loads).
  static_assert(BQ == 64, "one lane of the first wave per query row");
  float pl1 = 0.f, pl2 = 0.f, pg = 0.f, pkl = 0.f;
  auto fetch = [&](int st, int64_t q0) {
    tile_load_async<BQ, RB1>(sQ1(st), q1p, p.sq1.n * ESZ, (int)q0, (int)p.NQ, wave, lane);
    tile_load_async<BQ, RB2>(sQ2(st), q2p, p.sq2.n * ESZ, (int)q0, (int)p.NQ, wave, lane);
    if (wave == 0) {
      const int64_t q = q0 + lane;
      const int64_t o = bh * p.NQ + (q < p.NQ ? q : p.NQ - 1);  // rows past N_Q are zeroed at the stash
      pl1 = p.lse1[o];
      pl2 = p.lse2[o];
      pg = p.dkl[o];
      pkl = p.kl[o];
    }
  };
  auto stash = [&](int st, int64_t q0) {
    if (wave == 0) {
      const bool valid = q0 + lane < p.NQ;
      float A1 = kZeroRow, A2 = kZeroRow;
      if (valid) joint_row_consts(pl1, pl2, pg, A1, A2);
      float(*v)[BQ] = sVec(st);
      v[0][lane] = A1;
      v[1][lane] = A2;
      v[2][lane] = valid ? pkl : 0.f;
      v[3][lane] = (valid && pg < 0.f) ? -1.f : 1.f;
      const bool neg = __builtin_amdgcn_ballot_w64(valid && pg < 0.f) != 0;
      if (lane == 0) sNeg[st] = neg ? 1 : 0;
    }
  };

  if (nsteps > 0) {
    fetch(0, qbeg);
    stash(0, qbeg);
  }
  wait_vm();
  __syncthreads();
  const float c1 = p.c1, c2 = p.c2;
  const int prow = rperm(col);

  // One query step; the stage is a compile-time constant in the mask-free
  // steps (run in pairs), so it folds into the immediate offset of every
  // LDS read.
  auto step = [&](auto masked, auto stc, int64_t it) __attribute__((always_inline)) {
    const int st = stc;  // it & 1
    constexpr bool MASKED = decltype(masked)::value;
    const int64_t q0 = qbeg + it * BQ;
    if (it + 1 < nsteps) fetch(st ^ 1, q0 + BQ);
    const char* const tq1 = sQ1(st);
    const char* const tq2 = sQ2(st);
    const bool neg_tile = __builtin_amdgcn_readfirstlane(sNeg[st]) != 0;
    // Gradient work of query block qb from its logit accumulators.
    // Registers 8 run .. 8 run + 7 hold rows 32 qb + 16 run + 8 half + 0..7
    // (the rperm order): they form K chunk `run` (bf16) or chunks
    // 8 run .. 8 run + 7 (fp32) of both dK products.
    auto grad = [&](int qb, const f32x16& s1, const f32x16& s2) __attribute__((always_inline)) {
      const int64_t qb0 = q0 + 32 * qb;
      const bool need_mask = MASKED && ((qb0 + 32 > p.NQ) || (kw0 + 32 > p.NK) || (CAUSAL && kw0 + 31 > qb0 + off));
      const int qlim = clamp_i32(p.NQ - qb0), cmin = clamp_i32(key - qb0 - off);
#pragma unroll
      for (int run = 0; run < 2; ++run) {
        // Gradient operands read before the dS work, so their latency
        // overlaps it.
        frag bq1[NB1], bq2[NB2];
        if constexpr (EPL != 1) {
#pragma unroll
          for (int cb = 0; cb < NB1; ++cb) bq1[cb] = lds_tr_frag_swz<RB1>(tq1, 32 * qb + run * KC, 32 * cb, lane);
#pragma unroll
          for (int cb = 0; cb < NB2; ++cb) bq2[cb] = lds_tr_frag_swz<RB2>(tq2, 32 * qb + run * KC, 32 * cb, lane);
        }
        auto row8 = [&](int which, float (&dst)[8]) __attribute__((always_inline)) {
          const float4* v = reinterpret_cast<const float4*>(&sVec(st)[which][32 * qb + 16 * run + 8 * half]);
          const float4 y0 = v[0], y1 = v[1];
          dst[0] = y0.x; dst[1] = y0.y; dst[2] = y0.z; dst[3] = y0.w;
          dst[4] = y1.x; dst[5] = y1.y; dst[6] = y1.z; dst[7] = y1.w;
        };
        float a1[8], a2[8], kl8[8];
        row8(0, a1);
        row8(1, a2);
        row8(2, kl8);
        float ds1[8], ds2[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int r = 8 * run + i;
          dS_both_abs(s1[r], s2[r], c1, c2, a1[i], a2[i], kl8[i], ds1[i], ds2[i]);
        }
        if (neg_tile) {
          float sg[8];
          row8(3, sg);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            ds1[i] *= sg[i];
            ds2[i] *= sg[i];
          }
        }
        if (need_mask) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int ro = rloc(8 * run + i, half);
            const bool vis = kvalid && ro < qlim && (!CAUSAL || ro >= cmin);
            ds1[i] = vis ? ds1[i] : 0.f;
            ds2[i] = vis ? ds2[i] : 0.f;
          }
        }
        if constexpr (EPL == 1) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int c = 8 * run + i;
            const int qr = 32 * qb + rloc(c, half);
#pragma unroll
            for (int cb = 0; cb < NB1; ++cb)
              dk1[cb] = M::run(ds1[i], *reinterpret_cast<const float*>(&tq1[T1::off(qr, (32 * cb + col) * ESZ)]),
                               dk1[cb]);
#pragma unroll
            for (int cb = 0; cb < NB2; ++cb)
              dk2[cb] = M::run(ds2[i], *reinterpret_cast<const float*>(&tq2[T2::off(qr, (32 * cb + col) * ESZ)]),
                               dk2[cb]);
          }
        } else {
          frag a1f, a2f;
#pragma unroll
          for (int e = 0; e < EPL; ++e) {
            a1f[e] = from_f32<T>(ds1[e]);
            a2f[e] = from_f32<T>(ds2[e]);
          }
#pragma unroll
          for (int cb = 0; cb < NB1; ++cb) dk1[cb] = M::run(a1f, bq1[cb], dk1[cb]);
#pragma unroll
          for (int cb = 0; cb < NB2; ++cb) dk2[cb] = M::run(a2f, bq2[cb], dk2[cb]);
        }
      }
    };
    // Logits of query block qb.  bf16: all operand fragments are read before
    // the MFMA chains (one wave per SIMD: no other wave hides the LDS
    // latency); per-chunk LDS offsets are left to the compiler, which keeps
    // them as loop invariants (the stage folds into the immediate offset).
    auto read = [&](int qb, frag (&f1)[NC1], frag (&f2)[NC2]) __attribute__((always_inline)) {
      const int qrow = 32 * qb + prow;
#pragma unroll
      for (int c = 0; c < NC1; ++c) f1[c] = M::load(&tq1[T1::off(qrow, (c * KC + half * EPL) * ESZ)]);
#pragma unroll
      for (int c = 0; c < NC2; ++c) f2[c] = M::load(&tq2[T2::off(qrow, (c * KC + half * EPL) * ESZ)]);
    };
    auto chain = [&](const frag (&f1)[NC1], const frag (&f2)[NC2], f32x16& s1, f32x16& s2)
        __attribute__((always_inline)) {
#pragma unroll
      for (int c = 0; c < (NC1 > NC2 ? NC1 : NC2); ++c) {
        if (c < NC1) s1 = M::run(f1[c], kf1[c], s1);
        if (c < NC2) s2 = M::run(f2[c], kf2[c], s2);
      }
    };
    static_assert(BQ == 64, "the step pipeline below assumes two 32-row query blocks per tile");
    if constexpr (EPL != 1 && !MASKED) {
      // Mask-free step, software-pipelined over its two query blocks: block
      // 1's reads are issued right after block 0's MFMA chains, so their
      // latency hides behind block 0's dS work, with which block 1's MFMAs
      // can then interleave.
      f32x16 s1a = f32x16{}, s2a = f32x16{}, s1b = f32x16{}, s2b = f32x16{};
      frag fa1[NC1], fa2[NC2], fb1[NC1], fb2[NC2];
      read(0, fa1, fa2);
      __builtin_amdgcn_sched_barrier(0);
      chain(fa1, fa2, s1a, s2a);
      read(1, fb1, fb2);
      __builtin_amdgcn_sched_barrier(0);
      chain(fb1, fb2, s1b, s2b);
      grad(0, s1a, s2a);
      grad(1, s1b, s2b);
    } else {
#pragma unroll
      for (int qb = 0; qb < BQ / 32; ++qb) {
        const int64_t qb0 = q0 + 32 * qb;
        if (MASKED && (kw0 >= p.NK || qb0 >= p.NQ || (CAUSAL && kw0 > qb0 + 31 + off))) continue;  // fully masked
        f32x16 s1 = f32x16{}, s2 = f32x16{};
        if constexpr (EPL == 1) {
          const int qrow = 32 * qb + prow;
#pragma unroll
          for (int c = 0; c < NC1; ++c)
            s1 = M::run(M::load(&tq1[T1::off(qrow, (c * KC + half * EPL) * ESZ)]), kf1[c], s1);
#pragma unroll
          for (int c = 0; c < NC2; ++c)
            s2 = M::run(M::load(&tq2[T2::off(qrow, (c * KC + half * EPL) * ESZ)]), kf2[c], s2);
        } else {
          frag f1[NC1], f2[NC2];
          read(qb, f1, f2);
          __builtin_amdgcn_sched_barrier(0);  // keep every read ahead of the MFMA chains
          chain(f1, f2, s1, s2);
        }
        grad(qb, s1, s2);
      }
    }
    if (it + 1 < nsteps) stash(st ^ 1, q0 + BQ);
    wait_vm();
    __syncthreads();
  };
  // Steps [0, head) reach the causal diagonal, [tail, nsteps) the ragged
  // query edge; a ragged key tile masks every step.
  int64_t head = 0, tail = nsteps;
  if (kt0 + kBwdBK > p.NK) {
    head = nsteps;
  } else {
    const int64_t x = kt0 + kBwdBK - 1 - off - qbeg;
    if (CAUSAL && x > 0) head = min(nsteps, (x + BQ - 1) / BQ);
    if (p.NQ % BQ != 0) tail = max(head, nsteps - 1);
  }
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  int64_t it = 0;
  for (; it < head; ++it) step(std::true_type{}, (int)(it & 1), it);
  if constexpr (EPL != 1) {
    // (fp32 keeps one step per iteration: the unrolled pair spills there.)
    if (it < tail && (it & 1)) {
      step(std::false_type{}, I1{}, it);
      ++it;
    }
    for (; it + 1 < tail; it += 2) {
      step(std::false_type{}, I0{}, it);
      step(std::false_type{}, I1{}, it + 1);
    }
  }
  for (; it < tail; ++it) step(std::false_type{}, (int)(it & 1), it);
  for (; it < nsteps; ++it) step(std::true_type{}, (int)(it & 1), it);

  char* const dk1p = (char*)p.dk + (b * p.sdk.b + h * p.sdk.h) * ESZ;
  char* const dk2p = (char*)p.dk_s + (b * p.sdk_s.b + h * p.sdk_s.h) * ESZ;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int64_t kk = kw0 + acc_row(r, half);
    if (kk < p.NK) {
#pragma unroll
      for (int cb = 0; cb < NB1; ++cb)
        *reinterpret_cast<T*>(dk1p + (kk * p.sdk.n + 32 * cb + col) * ESZ) = from_f32<T>(dk1[cb][r] * p.scale_g);
#pragma unroll
      for (int cb = 0; cb < NB2; ++cb)
        *reinterpret_cast<T*>(dk2p + (kk * p.sdk_s.n + 32 * cb + col) * ESZ) = from_f32<T>(dk2[cb][r] * p.scale_s);
    }
  }
}

// ---------------------------------------------------------------------------
// Joint dQ kernel: 4 waves own 128 queries (32 each) of one (b, h) and stream
// the 64-key tiles they see.  Per 32-key block each wave forms Sᵀ = K Qᵀ
// (query = accumulator column, Q in registers), both dS with per-lane row
// constants, dQ1 += dS1 K1 and dQ2 += dS2 K2.
// ---------------------------------------------------------------------------
template <typename T, int D1, int D2, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void bwd_joint_dq_kernel(const BwdParams p) {
  using M = Mfma<T>;
  using frag = typename M::frag;
  constexpr int KC = M::KC, EPL = M::EPL;
  constexpr int NC1 = D1 / KC, NC2 = D2 / KC;
  constexpr int NB1 = D1 / 32, NB2 = D2 / 32;
  constexpr int ESZ = sizeof(T);
  constexpr int BQ = 128, BK = kDqBK;
  constexpr int RB1 = D1 * ESZ, RB2 = D2 * ESZ;  // bytes per key row
  using T1 = SwzTile<RB1>;
  using T2 = SwzTile<RB2>;

  __shared__ __attribute__((aligned(1024))) char sK1a[BK * RB1], sK1b[BK * RB1];
  __shared__ __attribute__((aligned(1024))) char sK2a[BK * RB2], sK2b[BK * RB2];
  auto sK1 = [&](int st) __attribute__((always_inline)) -> char* { return st ? sK1b : sK1a; };
  auto sK2 = [&](int st) __attribute__((always_inline)) -> char* { return st ? sK2b : sK2a; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int half = lane >> 5, col = lane & 31;

  const int num_qtiles = (int)((p.NQ + BQ - 1) / BQ);
  const int64_t t = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t bh = t / num_qtiles;
  int qt = (int)(t % num_qtiles);
  if (CAUSAL) qt = num_qtiles - 1 - qt;  // longest rows first
  const int64_t b = bh / p.H, h = bh % p.H;
  const int64_t off = p.NK - p.NQ;
  const int64_t qw0 = (int64_t)qt * BQ + 32 * wave;
  const int64_t qi = qw0 + col;
  const bool qvalid = qi < p.NQ;

  const char* const q1p = (const char*)p.q1 + (b * p.sq1.b + h * p.sq1.h) * ESZ;
  const char* const q2p = (const char*)p.q2 + (b * p.sq2.b + h * p.sq2.h) * ESZ;
  const char* const k1p = (const char*)p.k1 + (b * p.sk1.b + h * p.sk1.h) * ESZ;
  const char* const k2p = (const char*)p.k2 + (b * p.sk2.b + h * p.sk2.h) * ESZ;

  frag qf1[NC1], qf2[NC2];
#pragma unroll
  for (int c = 0; c < NC1; ++c)
    qf1[c] = qvalid ? M::load(q1p + (qi * p.sq1.n + c * KC + half * EPL) * ESZ) : M::zero();
#pragma unroll
  for (int c = 0; c < NC2; ++c)
    qf2[c] = qvalid ? M::load(q2p + (qi * p.sq2.n + c * KC + half * EPL) * ESZ) : M::zero();

  // Row constants of this lane's query row (see dS_both_abs); the sign of g
  // multiplies the finished dQ rows.
  float A1 = kZeroRow, A2 = kZeroRow, klr = 0.f;
  if (qvalid) {
    const int64_t o = bh * p.NQ + qi;
    joint_row_consts(p.lse1[o], p.lse2[o], p.dkl[o], A1, A2);
    klr = p.kl[o];
  }

  f32x16 dq1[NB1], dq2[NB2];
#pragma unroll
  for (int cb = 0; cb < NB1; ++cb) dq1[cb] = f32x16{};
#pragma unroll
  for (int cb = 0; cb < NB2; ++cb) dq2[cb] = f32x16{};

  int64_t kend = p.NK;
  if (CAUSAL) kend = min(kend, (int64_t)(qt + 1) * BQ + off);
  const int64_t nsteps = kend > 0 ? (kend + BK - 1) / BK : 0;
  const int64_t wave_kmax = CAUSAL ? qw0 + 31 + off : p.NK - 1;

  // A full key tile's direct-to-LDS loads take a wave-uniform base (scalar
  // registers) plus one loop-invariant 32-bit lane offset per side (the
  // swizzle repeats every 16 rows, so all of a wave's instructions share it);
  // the ragged last tile takes the clamping loader.
  const int64_t rs1 = p.sk1.n * ESZ, rs2 = p.sk2.n * ESZ;
  constexpr int RPI1 = 1024 / RB1, RPI2 = 1024 / RB2;  // rows per load instruction
  const int r01 = wave * RPI1 + lane / T1::CPR, r02 = wave * RPI2 + lane / T2::CPR;
  const unsigned lo1 = (unsigned)(r01 * (int)rs1 + (((lane % T1::CPR) ^ T1::swz(r01)) * 16));
  const unsigned lo2 = (unsigned)(r02 * (int)rs2 + (((lane % T2::CPR) ^ T2::swz(r02)) * 16));
  auto fetch = [&](int st, int64_t j0) {
    if (j0 + BK <= p.NK) {
      unsigned o1 = lo1, o2 = lo2;
      asm volatile("" : "+v"(o1), "+v"(o2));  // keep the offsets 32-bit (see the forward kernel)
#pragma unroll
      for (int k = 0; k < BK / RPI1 / 4; ++k)
        global_load_lds16(uniform_ptr(k1p + (j0 + 4 * k * RPI1) * rs1) + o1, sK1(st) + (wave + 4 * k) * 1024);
#pragma unroll
      for (int k = 0; k < BK / RPI2 / 4; ++k)
        global_load_lds16(uniform_ptr(k2p + (j0 + 4 * k * RPI2) * rs2) + o2, sK2(st) + (wave + 4 * k) * 1024);
    } else {
      tile_load_async<BK, RB1>(sK1(st), k1p, rs1, (int)j0, (int)p.NK, wave, lane);
      tile_load_async<BK, RB2>(sK2(st), k2p, rs2, (int)j0, (int)p.NK, wave, lane);
    }
  };

  if (nsteps > 0) fetch(0, 0);
  wait_vm();
  __syncthreads();
  const float c1 = p.c1, c2 = p.c2;
  const int prow = rperm(col);

  auto step = [&](auto masked, auto stc, int64_t it) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked)::value;
    const int st = stc;  // it & 1; a compile-time constant in the mask-free steps
    const int64_t j0 = it * BK;
    if (it + 1 < nsteps) fetch(st ^ 1, j0 + BK);
    const char* const tk1 = sK1(st);
    const char* const tk2 = sK2(st);

    if (!MASKED || wave_uniform(j0 <= wave_kmax)) {
      const bool need_mask =
          MASKED && wave_uniform((j0 + BK > p.NK) || (CAUSAL && j0 + BK - 1 > qw0 + off) || (qw0 + 32 > p.NQ));
      // Gradient work of block kb from its logit accumulators.
      auto grad = [&](int kb, const f32x16& s1, const f32x16& s2) __attribute__((always_inline)) {
        const int klim = clamp_i32(p.NK - (j0 + kb * 32)), cmax = clamp_i32(qi + off - (j0 + kb * 32));
        // Registers 8 run .. 8 run + 7 hold keys kb 32 + 16 run + 8 half + 0..7.
#pragma unroll
        for (int run = 0; run < 2; ++run) {
          // Gradient operands read before the dS work.
          frag bk1[NB1], bk2[NB2];
          if constexpr (EPL != 1) {
#pragma unroll
            for (int cb = 0; cb < NB1; ++cb) bk1[cb] = lds_tr_frag_swz<RB1>(tk1, kb * 32 + run * KC, 32 * cb, lane);
#pragma unroll
            for (int cb = 0; cb < NB2; ++cb) bk2[cb] = lds_tr_frag_swz<RB2>(tk2, kb * 32 + run * KC, 32 * cb, lane);
          }
          float ds1[8], ds2[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int r = 8 * run + i;
            dS_both_abs(s1[r], s2[r], c1, c2, A1, A2, klr, ds1[i], ds2[i]);
          }
          if (need_mask) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const int ro = rloc(8 * run + i, half);
              const bool vis = qvalid && ro < klim && (!CAUSAL || ro <= cmax);
              ds1[i] = vis ? ds1[i] : 0.f;
              ds2[i] = vis ? ds2[i] : 0.f;
            }
          }
          if constexpr (EPL == 1) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const int kr = kb * 32 + rloc(8 * run + i, half);
#pragma unroll
              for (int cb = 0; cb < NB1; ++cb)
                dq1[cb] = M::run(ds1[i], *reinterpret_cast<const float*>(&tk1[T1::off(kr, (32 * cb + col) * ESZ)]),
                                 dq1[cb]);
#pragma unroll
              for (int cb = 0; cb < NB2; ++cb)
                dq2[cb] = M::run(ds2[i], *reinterpret_cast<const float*>(&tk2[T2::off(kr, (32 * cb + col) * ESZ)]),
                                 dq2[cb]);
            }
          } else {
            frag a1, a2;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
              a1[e] = from_f32<T>(ds1[e]);
              a2[e] = from_f32<T>(ds2[e]);
            }
#pragma unroll
            for (int cb = 0; cb < NB1; ++cb)
              dq1[cb] = M::run(a1, bk1[cb], dq1[cb]);
#pragma unroll
            for (int cb = 0; cb < NB2; ++cb) dq2[cb] = M::run(a2, bk2[cb], dq2[cb]);
          }
        }
      };
      static_assert(BK == 64, "the step pipeline below assumes two 32-key blocks per tile");
      if constexpr (EPL != 1) {
        // Software pipeline over the tile's two blocks: all operand fragments
        // of a block are read before its MFMA chains (one wave per SIMD: no
        // other wave hides the LDS latency), and block 1's reads are issued
        // right after block 0's chains, so their latency hides behind block
        // 0's dS work, with which block 1's MFMAs can then interleave.
        auto read = [&](int kb, frag (&f1)[NC1], frag (&f2)[NC2]) __attribute__((always_inline)) {
          const int krow = kb * 32 + prow;
#pragma unroll
          for (int c = 0; c < NC1; ++c) f1[c] = M::load(&tk1[T1::off(krow, (c * KC + half * EPL) * ESZ)]);
#pragma unroll
          for (int c = 0; c < NC2; ++c) f2[c] = M::load(&tk2[T2::off(krow, (c * KC + half * EPL) * ESZ)]);
        };
        auto chain = [&](const frag (&f1)[NC1], const frag (&f2)[NC2], f32x16& s1, f32x16& s2)
            __attribute__((always_inline)) {
#pragma unroll
          for (int c = 0; c < (NC1 > NC2 ? NC1 : NC2); ++c) {
            if (c < NC1) s1 = M::run(f1[c], qf1[c], s1);
            if (c < NC2) s2 = M::run(f2[c], qf2[c], s2);
          }
        };
        f32x16 s1a = f32x16{}, s2a = f32x16{}, s1b = f32x16{}, s2b = f32x16{};
        frag fa1[NC1], fa2[NC2], fb1[NC1], fb2[NC2];
        read(0, fa1, fa2);
        __builtin_amdgcn_sched_barrier(0);
        chain(fa1, fa2, s1a, s2a);
        read(1, fb1, fb2);
        __builtin_amdgcn_sched_barrier(0);
        chain(fb1, fb2, s1b, s2b);
        grad(0, s1a, s2a);
        grad(1, s1b, s2b);
      } else {
#pragma unroll
        for (int kb = 0; kb < BK / 32; ++kb) {
          f32x16 s1 = f32x16{}, s2 = f32x16{};
          const int krow = kb * 32 + prow;
#pragma unroll
          for (int c = 0; c < NC1; ++c)
            s1 = M::run(M::load(&tk1[T1::off(krow, (c * KC + half * EPL) * ESZ)]), qf1[c], s1);
#pragma unroll
          for (int c = 0; c < NC2; ++c)
            s2 = M::run(M::load(&tk2[T2::off(krow, (c * KC + half * EPL) * ESZ)]), qf2[c], s2);
          grad(kb, s1, s2);
        }
      }
    }
    wait_vm();
    __syncthreads();
  };
  // Steps [tail, nsteps) reach the causal diagonal of some wave or the ragged
  // key edge; a ragged query tile masks all (see bwd_split.hip).
  auto first_ge = [&](int64_t x) -> int64_t { return x <= 0 ? 0 : (x + BK - 1) / BK; };
  int64_t tail = 0;
  if ((int64_t)qt * BQ + BQ <= p.NQ) {
    tail = min(nsteps, first_ge(p.NK - BK + 1));
    if (CAUSAL) tail = min(tail, first_ge((int64_t)qt * BQ + off - BK + 2));
  }
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  int64_t it = 0;
  if constexpr (EPL != 1) {
    // (fp32 keeps one step per iteration: the unrolled pair spills there.)
    for (; it + 1 < tail; it += 2) {
      step(std::false_type{}, I0{}, it);
      step(std::false_type{}, I1{}, it + 1);
    }
  }
  for (; it < tail; ++it) step(std::false_type{}, (int)(it & 1), it);
  for (; it < nsteps; ++it) step(std::true_type{}, (int)(it & 1), it);

  char* const dq1p = (char*)p.dq + (b * p.sdq.b + h * p.sdq.h) * ESZ;
  char* const dq2p = (char*)p.dq_s + (b * p.sdq_s.b + h * p.sdq_s.h) * ESZ;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int64_t q = qw0 + acc_row(r, half);
    if (q < p.NQ) {
      const bool neg = p.dkl[bh * p.NQ + q] < 0.f;
      const float sc1 = neg ? -p.scale_g : p.scale_g, sc2 = neg ? -p.scale_s : p.scale_s;
#pragma unroll
      for (int cb = 0; cb < NB1; ++cb)
        *reinterpret_cast<T*>(dq1p + (q * p.sdq.n + 32 * cb + col) * ESZ) = from_f32<T>(dq1[cb][r] * sc1);
#pragma unroll
      for (int cb = 0; cb < NB2; ++cb)
        *reinterpret_cast<T*>(dq2p + (q * p.sdq_s.n + 32 * cb + col) * ESZ) = from_f32<T>(dq2[cb][r] * sc2);
    }
  }
}

namespace {

template <typename T, int D1, int D2, bool C>
hipError_t run_joint(const BwdParams& p, int64_t BH, hipStream_t s, void (*between)(hipStream_t)) {
  const int64_t gk = BH * p.num_ktiles;
  hipLaunchKernelGGL((bwd_joint_dk_kernel<T, D1, D2, C>), dim3((unsigned)gk), dim3(kThreads), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (between) between(s);
  const int64_t gq = BH * ((p.NQ + 127) / 128);
  hipLaunchKernelGGL((bwd_joint_dq_kernel<T, D1, D2, C>), dim3((unsigned)gq), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

template <typename T, int D1, int D2>
hipError_t joint_dims(const BwdParams& p, bool causal, int64_t BH, hipStream_t s, void (*bw)(hipStream_t)) {
  return causal ? run_joint<T, D1, D2, true>(p, BH, s, bw) : run_joint<T, D1, D2, false>(p, BH, s, bw);
}

template <typename T>
hipError_t joint_type(const BwdParams& p, int d1, int d2, bool causal, int64_t BH, hipStream_t s,
                      void (*bw)(hipStream_t)) {
  if (d1 == 128 && d2 == 128) return joint_dims<T, 128, 128>(p, causal, BH, s, bw);
  if (d1 == 128 && d2 == 64) return joint_dims<T, 128, 64>(p, causal, BH, s, bw);
  if (d1 == 64 && d2 == 128) return joint_dims<T, 64, 128>(p, causal, BH, s, bw);
  if (d1 == 64 && d2 == 64) return joint_dims<T, 64, 64>(p, causal, BH, s, bw);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_backward_joint(const BwdParams& p, int dtype, int d1, int d2, bool causal, int64_t BH,
                                 hipStream_t s, void (*between)(hipStream_t)) {
  if (dtype == 0) return joint_type<bf16>(p, d1, d2, causal, BH, s, between);
  return joint_type<float>(p, d1, d2, causal, BH, s, between);
}

}  // namespace skl
