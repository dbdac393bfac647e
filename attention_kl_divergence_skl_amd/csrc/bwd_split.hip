// Atomic-free backward of the attention-KL primitive for gfx950: one kernel
// owns keys and accumulates dK, one owns queries and accumulates dQ.
//
// Recompute-based (agidaily.cc StreamKL article, section "Backward:
// recompute-based tile-by-tile gradients"): P_k = 2^(t_k - LSE_k log2 e) is
// rebuilt from the saved LSEs tile by tile; for the two gradient settings
//   student (optimise P2):  dS2 = g (P2 - P1)
//   teacher (optimise P1):  dS1 = g P1 (r - KL),  r = ln2 ((t1 - L1) - (t2 - L2))
// with the log-ratio r taken from logits (an underflowed P1 gives an exact 0).
//
// Why two kernels.  The pages fuse dQ and dK in one kernel with atomic dQ
// updates (section "GPU kernel optimisations").  On MI355X the L2 executes
// fp32 atomics at about one element per channel per clock, so the ~7e10 dQ
// atomics of a causal 64K x 32-head backward cost more than recomputing the
// two logit tiles once more; here each kernel writes its gradient once, with
// plain stores, and the result is bitwise deterministic.  (The fused kernel
// remains available as SKL_BWD_FUSED_ATOMIC.)
//
// When the query tiles alone are too few to fill the GPU (few heads and
// queries, many keys) the dQ kernel also cuts its keys into tile-aligned
// ranges: each (query tile, key range) workgroup writes an unscaled fp32
// partial and convert_kernel sums them in a fixed order, so the result stays
// deterministic.
//
// Both kernels form logits with the rows of the streamed operand loaded in
// the rperm order, so an accumulator register block is directly the A operand
// of the gradient MFMA; the other operand of that MFMA comes from a row-major
// LDS tile through gfx950 transposing reads (lds_tr_frag), so no transposed
// copy of anything is ever written.

#include <type_traits>

#include "skl_device.h"
#include "skl_internal.h"

namespace skl {

namespace {

// sign(g) dS of one accumulator element from the two logits (raw dot
// products) and two row constants that fold the upstream gradient into the
// exponents.  With
// u_k = t_k - LSE_k log2 e (so P_k = 2^u_k), ga = g (student) or g ln2
// (teacher) and k = log2 |ga|:
//   student: g (P2 - P1) = sign(g) (2^(u2 + k) - 2^(u1 + k))
//   teacher: g P1 (ln2 (u1 - u2) - KL)
//              = sign(g) 2^(u1 + k) ((u1 + k) - (u2 + k + KL log2 e))
// so the row constants are A1 = L1 - k and A2 = L2 - k (student) or
// L2 - k - KL log2 e (teacher), and the element needs no multiply by g.  A
// row with g = 0 gets A1 = kZeroRow (and a finite A2), whose exponential is 0.
// The dQ kernel (one query per lane) applies the sign to each finished dQ
// row; the dK kernel (whose accumulator rows are queries) multiplies dS by it
// in the tiles that have a row with g < 0.
template <bool TEACHER>
__device__ __forceinline__ float dS_abs(float s1, float s2, float c1, float c2, float A1, float A2) {
  const float w1 = fmaf(s1, c1, -A1);
  const float w2 = fmaf(s2, c2, -A2);
  if (TEACHER) return exp2_hw(w1) * (w1 - w2);
  return exp2_hw(w2) - exp2_hw(w1);
}

constexpr float kZeroRow = 1e30f;

// Row constants of dS_abs from the saved row values (natural-log LSEs, KL and
// g); valid rows only.
template <bool TEACHER>
__device__ __forceinline__ void row_consts(float lse1, float lse2, float kl, float g, float& A1, float& A2) {
  const float ga = TEACHER ? g * kLn2 : g;
  if (ga == 0.f) {
    A1 = kZeroRow;
    A2 = TEACHER ? 0.f : kZeroRow;
    return;
  }
  const float k = log2f(fabsf(ga));
  A1 = fmaf(lse1, kLog2e, -k);
  A2 = TEACHER ? fmaf(lse2 - kl, kLog2e, -k) : fmaf(lse2, kLog2e, -k);
}

}  // namespace

// ---------------------------------------------------------------------------
// dK kernel: 4 waves own 128 keys (32 each) of one (b, h) and walk the query
// tiles of 64 rows that see them, 32 rows at a time.  Per block each wave forms
// S = Q Kᵀ (32 queries x its 32 keys; key = accumulator column, K in
// registers), dS in fp32, and dK += dSᵀ Q_g with dSᵀ straight from the
// accumulator registers and Q_g from the LDS query tile.  Query tiles are
// loaded straight into a double-buffered, swizzled LDS ring.
// ---------------------------------------------------------------------------
template <typename T, int D1, int D2, bool CAUSAL, bool TEACHER>
__global__ __launch_bounds__(kThreads, sizeof(T) == 2 ? 2 : 1) void bwd_dk_kernel(const BwdParams p) {
  using M = Mfma<T>;
  using frag = typename M::frag;
  constexpr int KC = M::KC, EPL = M::EPL;
  constexpr int NC1 = D1 / KC, NC2 = D2 / KC;
  constexpr int DG = TEACHER ? D1 : D2;
  constexpr int NCB = DG / 32;
  constexpr int ESZ = sizeof(T);
  constexpr int BQ = kDkBQ;
  constexpr int RB1 = D1 * ESZ, RB2 = D2 * ESZ;  // bytes per query row
  constexpr int RBG = TEACHER ? RB1 : RB2;
  using T1 = SwzTile<RB1>;
  using T2 = SwzTile<RB2>;
  using TG = SwzTile<RBG>;

  // The ring's two stages stay one [2][...] array here: as separate variables
  // (which lets the compiler see that reads of one stage do not wait for the
  // loads in flight into the other, as in the forward and dQ kernels) this
  // kernel spills heavily at 256 VGPRs, and measured slower.
  __shared__ __attribute__((aligned(1024))) char sQ1x[2][BQ * RB1];
  __shared__ __attribute__((aligned(1024))) char sQ2x[2][BQ * RB2];
  // Per query row of a tile: A1, A2 (row constants of dS_abs) and sign(g);
  // plus a flag per stage: some row of the tile has g < 0.
  __shared__ __attribute__((aligned(16))) float sVa[3][BQ], sVb[3][BQ];
  __shared__ int sNeg[2];
  auto sQ1 = [&](int st) __attribute__((always_inline)) -> char* { return sQ1x[st]; };
  auto sQ2 = [&](int st) __attribute__((always_inline)) -> char* { return sQ2x[st]; };
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

  f32x16 dk[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) dk[cb] = f32x16{};

  int64_t qbeg = 0;
  if (CAUSAL) qbeg = max((int64_t)0, kt0 - off) / BQ * BQ;
  const int64_t nsteps = (p.NQ - qbeg + BQ - 1) / BQ;

  // Query tiles go straight into a double-buffered LDS ring (loads of step
  // i+1 in flight during step i).  The row values of the tile (LSE1, LSE2, g
  // and, for the teacher, KL) are loaded by the first wave, one row per lane;
  // the fetch only loads them: any arithmetic on a loaded value would make the
  // wave wait for all its outstanding loads, the next tile's included, in the
  // middle of the step, so the row constants are formed at the stash after
  // the step.  |g| goes into the exponents (see dS_abs); its sign multiplies
  // dS only in the rare tiles that have a row with g < 0.
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
      if (TEACHER) pkl = p.kl[o];
    }
  };
  auto stash = [&](int st, int64_t q0) {
    if (wave == 0) {
      const bool valid = q0 + lane < p.NQ;
      float A1 = kZeroRow, A2 = TEACHER ? 0.f : kZeroRow;
      if (valid) row_consts<TEACHER>(pl1, pl2, pkl, pg, A1, A2);
      float(*v)[BQ] = sVec(st);
      v[0][lane] = A1;
      v[1][lane] = A2;
      v[2][lane] = (valid && pg < 0.f) ? -1.f : 1.f;
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
  // LDS address base of the gradient operand (bf16 tiles; unused in fp32).
  const SwzAddr<RBG> adg(prow, half, lane);

  // One query step.  The stage (which LDS buffer) is a template constant so
  // the buffer address folds into the immediate offset of every LDS read;
  // MASKED steps are those whose 64 x 128 (query, key) rectangle reaches past
  // the causal diagonal or a ragged edge, decided from workgroup-uniform
  // values, so the common unmasked step carries no mask code at all.
  auto step = [&](auto masked, auto stc, int64_t it) __attribute__((always_inline)) {
    const int st = stc;  // it & 1; a compile-time constant in the unrolled mask-free loop
    constexpr bool MASKED = decltype(masked)::value;
    const int64_t q0 = qbeg + it * BQ;
    if (it + 1 < nsteps) fetch(st ^ 1, q0 + BQ);  // next tile in flight during this step

    const char* qgs = TEACHER ? sQ1(st) : sQ2(st);  // gradient operand tile of this stage
    const bool neg_tile = __builtin_amdgcn_readfirstlane(sNeg[st]) != 0;
#pragma unroll
    for (int qb = 0; qb < BQ / 32; ++qb) {
      const int64_t qb0 = q0 + 32 * qb;
      if (MASKED && (kw0 >= p.NK || qb0 >= p.NQ || (CAUSAL && kw0 > qb0 + 31 + off))) continue;  // fully masked
      f32x16 s1 = f32x16{}, s2 = f32x16{};
      __builtin_amdgcn_s_setprio(1);  // MFMA burst at raised priority (as in the forward)
      // Logit operands: per-chunk LDS offsets left to the compiler (kept as
      // loop invariants; measured faster here than forming them at each
      // read), the gradient operands below through SwzAddr.
      // The two chains alternate, so each MFMA's predecessor in its chain is
      // two issues back.
      const int qrow = 32 * qb + prow;
      // The operands of chunk c + 1 are read while chunk c's MFMAs issue,
      // the order pinned by a scheduling barrier (the compiler otherwise
      // issues each pair of reads just before its MFMAs and waits on them).
      constexpr int NCM = NC1 > NC2 ? NC1 : NC2;
      frag pa1[2], pa2[2];
      auto ld = [&](int c, int slot) __attribute__((always_inline)) {
        if (c < NC1) pa1[slot] = M::load(&sQ1(st)[T1::off(qrow, (c * KC + half * EPL) * ESZ)]);
        if (c < NC2) pa2[slot] = M::load(&sQ2(st)[T2::off(qrow, (c * KC + half * EPL) * ESZ)]);
      };
      ld(0, 0);
#pragma unroll
      for (int c = 0; c < NCM; ++c) {
        if (c + 1 < NCM) ld(c + 1, (c + 1) & 1);
        __builtin_amdgcn_sched_barrier(0);
        if (c < NC1) s1 = M::run(pa1[c & 1], kf1[c], s1);
        if (c < NC2) s2 = M::run(pa2[c & 1], kf2[c], s2);
      }

      __builtin_amdgcn_s_setprio(0);
      // Registers 8 run .. 8 run + 7 hold rows 32 qb + 16 run + 8 half + 0..7:
      // their row constants are two float4 reads, and they form K chunk
      // `run` (bf16) or chunks 8 run .. 8 run + 7 (fp32) of dK += dSᵀ Q_g, so
      // each run is converted and consumed right away.
      // Within a masked step the mask is applied in one pass per run of 8
      // registers, under a per-lane condition (one exec-mask region per run).
      const bool need_mask = MASKED && ((qb0 + 32 > p.NQ) || (kw0 + 32 > p.NK) || (CAUSAL && kw0 + 31 > qb0 + off));
      // Row qb0 + ro sees this lane's key iff ro < NQ - qb0 and (causal) ro >= key - qb0 - off.
      const int qlim = clamp_i32(p.NQ - qb0), cmin = clamp_i32(key - qb0 - off);
#pragma unroll
      for (int run = 0; run < 2; ++run) {
        // The gradient operand's transposing reads are issued before the dS
        // work, so their latency overlaps it instead of stalling each
        // gradient MFMA (teacher -4%, student -2.8%, despite a few more
        // spilled registers in the student kernel).
        frag bq[NCB];
        if constexpr (EPL != 1) {
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) bq[cb] = adg.trfrag(qgs, (32 * qb + run * KC) * RBG, cb);
          __builtin_amdgcn_sched_barrier(0);
        }
        auto row8 = [&](int which, float (&dst)[8]) __attribute__((always_inline)) {
          const float4* v = reinterpret_cast<const float4*>(&sVec(st)[which][32 * qb + 16 * run + 8 * half]);
          const float4 x0 = v[0], x1 = v[1];
          dst[0] = x0.x; dst[1] = x0.y; dst[2] = x0.z; dst[3] = x0.w;
          dst[4] = x1.x; dst[5] = x1.y; dst[6] = x1.z; dst[7] = x1.w;
        };
        float a1[8], a2[8];
        row8(0, a1);
        row8(1, a2);
        float ds[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int r = 8 * run + i;
          ds[i] = dS_abs<TEACHER>(s1[r], s2[r], c1, c2, a1[i], a2[i]);
        }
        if (neg_tile) {
          float sg[8];
          row8(2, sg);
#pragma unroll
          for (int i = 0; i < 8; ++i) ds[i] *= sg[i];
        }
        if (need_mask) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int ro = rloc(8 * run + i, half);
            ds[i] = (kvalid && ro < qlim && (!CAUSAL || ro >= cmin)) ? ds[i] : 0.f;
          }
        }
        if constexpr (EPL == 1) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int c = 8 * run + i;
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
              const float bq = *reinterpret_cast<const float*>(qgs + TG::off(32 * qb + rloc(c, half), (32 * cb + col) * ESZ));
              dk[cb] = M::run(ds[i], bq, dk[cb]);
            }
          }
        } else {
          frag a;
#pragma unroll
          for (int e = 0; e < EPL; ++e) a[e] = from_f32<T>(ds[e]);
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
            dk[cb] = M::run(a, bq[cb], dk[cb]);
        }
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
    // step it is masked iff qbeg + it BQ < kt0 + kBwdBK - 1 - off =: x
    const int64_t x = kt0 + kBwdBK - 1 - off - qbeg;
    if (CAUSAL && x > 0) head = min(nsteps, (x + BQ - 1) / BQ);
    if (p.NQ % BQ != 0) tail = max(head, nsteps - 1);
  }
  int64_t it = 0;
  for (; it < head; ++it) step(std::true_type{}, (int)(it & 1), it);
  // Mask-free steps in stage pairs: the LDS stage is then a constant and
  // folds into the immediate offset of every LDS read.
  if (it < tail && (it & 1)) {
    step(std::false_type{}, 1, it);
    ++it;
  }
  for (; it + 1 < tail; it += 2) {
    step(std::false_type{}, std::integral_constant<int, 0>{}, it);
    step(std::false_type{}, std::integral_constant<int, 1>{}, it + 1);
  }
  if (it < tail) {
    step(std::false_type{}, 0, it);
    ++it;
  }
  for (; it < nsteps; ++it) step(std::true_type{}, (int)(it & 1), it);

  char* const dkp = (char*)p.dk + (b * p.sdk.b + h * p.sdk.h) * ESZ;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t kk = kw0 + acc_row(r, half);
      if (kk < p.NK)
        *reinterpret_cast<T*>(dkp + (kk * p.sdk.n + 32 * cb + col) * ESZ) = from_f32<T>(dk[cb][r] * p.scale_g);
    }
}

// ---------------------------------------------------------------------------
// dQ kernel: 4 waves own 128 queries (32 each) of one (b, h) and stream the
// key tiles (64 keys) they see, like the forward.  Per 32-key block each wave
// forms Sᵀ = K Qᵀ (query = accumulator column, Q in registers, K rows loaded
// in rperm order), dS in fp32 with per-lane row constants, and
// dQ += dS K_g with dS straight from the accumulator registers and K_g from
// the LDS key tile.  Key tiles are double-buffered in LDS.
// ---------------------------------------------------------------------------
template <typename T, int D1, int D2, bool CAUSAL, bool TEACHER>
__global__ __launch_bounds__(kThreads, sizeof(T) == 2 ? 2 : 1) void bwd_dq_kernel(const BwdParams p) {
  using M = Mfma<T>;
  using frag = typename M::frag;
  constexpr int KC = M::KC, EPL = M::EPL;
  constexpr int NC1 = D1 / KC, NC2 = D2 / KC;
  constexpr int DG = TEACHER ? D1 : D2;
  constexpr int NCB = DG / 32;
  constexpr int ESZ = sizeof(T);
  constexpr int BQ = 128, BK = kDqBK;
  constexpr int RB1 = D1 * ESZ, RB2 = D2 * ESZ;  // bytes per key row
  constexpr int RBG = TEACHER ? RB1 : RB2;
  using T1 = SwzTile<RB1>;
  using T2 = SwzTile<RB2>;
  using TG = SwzTile<RBG>;

  // Ring stages as separate LDS variables, so that the compiler can tell
  // reads of one stage from the direct-to-LDS loads in flight into the other
  // and does not wait for those loads before them.
  __shared__ __attribute__((aligned(1024))) char sK1a[BK * RB1], sK1b[BK * RB1];
  __shared__ __attribute__((aligned(1024))) char sK2a[BK * RB2], sK2b[BK * RB2];
  auto sK1 = [&](int st) __attribute__((always_inline)) -> char* { return st ? sK1b : sK1a; };
  auto sK2 = [&](int st) __attribute__((always_inline)) -> char* { return st ? sK2b : sK2a; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int half = lane >> 5, col = lane & 31;

  // Row and key indices are 32-bit (the host keeps N_Q and N_K below 2^30),
  // so the loop control below is scalar arithmetic.
  const int NQ = (int)p.NQ, NK = (int)p.NK;
  const int num_qtiles = (NQ + BQ - 1) / BQ;
  int64_t t = xcd_remap(blockIdx.x, gridDim.x);
  int split = 0;  // key range of this workgroup when the keys are split (few query tiles)
  if (p.dq_splits > 1) {
    split = (int)(t % p.dq_splits);
    t /= p.dq_splits;
  }
  const int64_t bh = t / num_qtiles;
  int qt = (int)(t % num_qtiles);
  if (CAUSAL) qt = num_qtiles - 1 - qt;  // longest rows first
  const int64_t b = bh / p.H, h = bh % p.H;
  const int off = NK - NQ;
  const int qw0 = qt * BQ + 32 * wave;
  const int qi = qw0 + col;
  const bool qvalid = qi < NQ;

  const char* const q1p = (const char*)p.q1 + (b * p.sq1.b + h * p.sq1.h) * ESZ;
  const char* const q2p = (const char*)p.q2 + (b * p.sq2.b + h * p.sq2.h) * ESZ;
  const char* const k1p = (const char*)p.k1 + (b * p.sk1.b + h * p.sk1.h) * ESZ;
  const char* const k2p = (const char*)p.k2 + (b * p.sk2.b + h * p.sk2.h) * ESZ;

  frag qf1[NC1], qf2[NC2];
#pragma unroll
  for (int c = 0; c < NC1; ++c)
    qf1[c] = qvalid ? M::load(q1p + ((int64_t)qi * p.sq1.n + c * KC + half * EPL) * ESZ) : M::zero();
#pragma unroll
  for (int c = 0; c < NC2; ++c)
    qf2[c] = qvalid ? M::load(q2p + ((int64_t)qi * p.sq2.n + c * KC + half * EPL) * ESZ) : M::zero();

  // Row constants of this lane's query row (see dS_abs).  The sign of g is
  // applied to the finished dQ row instead of to every element.
  float A1 = kZeroRow, A2 = TEACHER ? 0.f : kZeroRow;
  if (qvalid) {
    const int64_t o = bh * p.NQ + qi;
    row_consts<TEACHER>(p.lse1[o], p.lse2[o], TEACHER ? p.kl[o] : 0.f, p.dkl[o], A1, A2);
  }

  f32x16 dq[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) dq[cb] = f32x16{};

  int kbeg = 0, kend = NK;
  if (CAUSAL) kend = min(kend, (qt + 1) * BQ + off);
  if (p.dq_splits > 1) {
    kbeg = split * p.dq_split_len;
    kend = min(kend, kbeg + p.dq_split_len);
  }
  const int nsteps = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;
  const int wave_kmax = CAUSAL ? qw0 + 31 + off : NK - 1;

  auto fetch = [&](int st, int j0) {
    tile_load_async<BK, RB1>(sK1(st), k1p, p.sk1.n * ESZ, j0, NK, wave, lane);
    tile_load_async<BK, RB2>(sK2(st), k2p, p.sk2.n * ESZ, j0, NK, wave, lane);
  };

  if (nsteps > 0) fetch(0, kbeg);
  wait_vm();
  __syncthreads();
  const float c1 = p.c1, c2 = p.c2;
  const int prow = rperm(col);

  // One key step (64 keys).  MASKED steps are those that reach the causal
  // diagonal of some wave or a ragged edge; the others carry no mask code.
  auto step = [&](auto masked, auto stc, int it) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked)::value;
    const int st = stc;  // it & 1; a compile-time constant in the unrolled mask-free loop
    const int j0 = kbeg + it * BK;
    if (it + 1 < nsteps) fetch(st ^ 1, j0 + BK);

    if (!MASKED || j0 <= wave_kmax) {
      const bool need_mask = MASKED && ((j0 + BK > NK) || (CAUSAL && j0 + BK - 1 > qw0 + off) || (qw0 + 32 > NQ));
      // (Here the per-chunk LDS offsets are left to the compiler, which keeps
      // them as loop invariants: measured faster than forming them at each
      // read as the dK kernel does.)
      const char* kg = TEACHER ? sK1(st) : sK2(st);
#pragma unroll
      for (int kb = 0; kb < BK / 32; ++kb) {
        f32x16 s1 = f32x16{}, s2 = f32x16{};
        __builtin_amdgcn_s_setprio(1);  // MFMA burst at raised priority (as in the forward)
        // Key j0 + 32 kb + ro is visible iff ro < NK - jb and (causal) ro <= qi + off - jb.
        const int klim = NK - (j0 + kb * 32), cmax = qi + off - (j0 + kb * 32);
        const int krow = kb * 32 + prow;
#pragma unroll
        for (int c = 0; c < (NC1 > NC2 ? NC1 : NC2); ++c) {  // chains alternate (see the dK kernel)
          if (c < NC1) s1 = M::run(M::load(&sK1(st)[T1::off(krow, (c * KC + half * EPL) * ESZ)]), qf1[c], s1);
          if (c < NC2) s2 = M::run(M::load(&sK2(st)[T2::off(krow, (c * KC + half * EPL) * ESZ)]), qf2[c], s2);
        }
        __builtin_amdgcn_s_setprio(0);
        // Registers 8 run .. 8 run + 7 hold keys kb 32 + 16 run + 8 half + 0..7:
        // K chunk `run` (bf16) or chunks 8 run .. 8 run + 7 (fp32) of
        // dQ += dS K_g, consumed as soon as they are formed.
#pragma unroll
        for (int run = 0; run < 2; ++run) {
          float ds[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int r = 8 * run + i;
            ds[i] = dS_abs<TEACHER>(s1[r], s2[r], c1, c2, A1, A2);
          }
          if (need_mask) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const int ro = rloc(8 * run + i, half);
              ds[i] = (qvalid && ro < klim && (!CAUSAL || ro <= cmax)) ? ds[i] : 0.f;
            }
          }
          if constexpr (EPL == 1) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const int c = 8 * run + i;
#pragma unroll
              for (int cb = 0; cb < NCB; ++cb) {
                const float bk = *reinterpret_cast<const float*>(kg + TG::off(kb * 32 + rloc(c, half), (32 * cb + col) * ESZ));
                dq[cb] = M::run(ds[i], bk, dq[cb]);
              }
            }
          } else {
            frag a;
#pragma unroll
            for (int e = 0; e < EPL; ++e) a[e] = from_f32<T>(ds[e]);
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) dq[cb] = M::run(a, lds_tr_frag_swz<RBG>(kg, kb * 32 + run * KC, 32 * cb, lane), dq[cb]);
          }
        }
      }
    }
    wait_vm();
    __syncthreads();
  };
  // Steps [tail, nsteps) reach the causal diagonal of some wave (keys past
  // qt 128 + off - 63) or the ragged key edge; a ragged query tile masks all.
  // Both conditions hold from some step on; first_ge(x) is the first step
  // whose first key is >= x.
  auto first_ge = [&](int x) -> int { return x <= kbeg ? 0 : (x - kbeg + BK - 1) / BK; };
  int tail = 0;
  if (qt * BQ + BQ <= NQ) {
    tail = min(nsteps, first_ge(NK - BK + 1));
    if (CAUSAL) tail = min(tail, first_ge(qt * BQ + off - BK + 2));
  }
  int it = 0;
  // Mask-free steps in stage pairs (the LDS stage folds into the read offsets).
  for (; it + 1 < tail; it += 2) {
    step(std::false_type{}, std::integral_constant<int, 0>{}, it);
    step(std::false_type{}, std::integral_constant<int, 1>{}, it + 1);
  }
  if (it < tail) {
    step(std::false_type{}, 0, it);
    ++it;
  }
  for (; it < nsteps; ++it) step(std::true_type{}, it & 1, it);

  // dQ of this wave's rows: accumulator register r holds query qw0 + acc_row(r, half).
  if (p.dq_splits > 1) {
    // Unscaled fp32 partial of this key range (zeros for an empty range);
    // convert_kernel sums the ranges and applies the scale.
    const int64_t BH = gridDim.x / ((int64_t)num_qtiles * p.dq_splits);
    float* const dst = p.dq_part + ((int64_t)split * BH + bh) * p.NQ * DG;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t q = qw0 + acc_row(r, half);
        if (q < p.NQ) dst[q * DG + 32 * cb + col] = p.dkl[bh * p.NQ + q] < 0.f ? -dq[cb][r] : dq[cb][r];
      }
    return;
  }
  char* const dqp = (char*)p.dq + (b * p.sdq.b + h * p.sdq.h) * ESZ;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t q = qw0 + acc_row(r, half);
      if (q < p.NQ) {
        const float sc = p.dkl[bh * p.NQ + q] < 0.f ? -p.scale_g : p.scale_g;
        *reinterpret_cast<T*>(dqp + (q * p.sdq.n + 32 * cb + col) * ESZ) = from_f32<T>(dq[cb][r] * sc);
      }
    }
}

namespace {

template <typename T, int D1, int D2, bool C, bool TCH>
hipError_t run_split(const BwdParams& p, int64_t BH, hipStream_t s, void (*between)(hipStream_t)) {
  const int64_t gk = BH * p.num_ktiles;
  hipLaunchKernelGGL((bwd_dk_kernel<T, D1, D2, C, TCH>), dim3((unsigned)gk), dim3(kThreads), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (between) between(s);
  const int64_t gq = BH * ((p.NQ + 127) / 128) * (p.dq_splits > 1 ? p.dq_splits : 1);
  hipLaunchKernelGGL((bwd_dq_kernel<T, D1, D2, C, TCH>), dim3((unsigned)gq), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

template <typename T, int D1, int D2>
hipError_t split_dims(const BwdParams& p, bool causal, bool teacher, int64_t BH, hipStream_t s,
                      void (*bw)(hipStream_t)) {
  if (causal)
    return teacher ? run_split<T, D1, D2, true, true>(p, BH, s, bw) : run_split<T, D1, D2, true, false>(p, BH, s, bw);
  return teacher ? run_split<T, D1, D2, false, true>(p, BH, s, bw) : run_split<T, D1, D2, false, false>(p, BH, s, bw);
}

template <typename T>
hipError_t split_type(const BwdParams& p, int d1, int d2, bool causal, bool teacher, int64_t BH, hipStream_t s,
                      void (*bw)(hipStream_t)) {
  if (d1 == 128 && d2 == 128) return split_dims<T, 128, 128>(p, causal, teacher, BH, s, bw);
  if (d1 == 128 && d2 == 64) return split_dims<T, 128, 64>(p, causal, teacher, BH, s, bw);
  if (d1 == 64 && d2 == 128) return split_dims<T, 64, 128>(p, causal, teacher, BH, s, bw);
  if (d1 == 64 && d2 == 64) return split_dims<T, 64, 64>(p, causal, teacher, BH, s, bw);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_backward_split(const BwdParams& p, int dtype, int d1, int d2, bool causal, bool teacher,
                                 int64_t BH, hipStream_t s, void (*between)(hipStream_t)) {
  if (dtype == 0) return split_type<bf16>(p, d1, d2, causal, teacher, BH, s, between);
  return split_type<float>(p, d1, d2, causal, teacher, BH, s, between);
}

}  // namespace skl
