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
// Both kernels form logits with the rows of the streamed operand loaded in
// the rperm order, so an accumulator register block is directly the A operand
// of the gradient MFMA; the other operand of that MFMA comes from a row-major
// LDS tile through gfx950 transposing reads (lds_tr_frag), so no transposed
// copy of anything is ever written.

#include "skl_device.h"
#include "skl_internal.h"

namespace skl {

namespace {

constexpr int kPad = 32;  // LDS row pad (bytes): conflict-free 16-byte and transposing reads

// dS of one accumulator element from the two logits (raw dot products).
template <bool TEACHER>
__device__ __forceinline__ float dS_of(float s1, float s2, float c1, float c2, float L1, float L2, float g,
                                       float kl) {
  const float u1 = fmaf(s1, c1, -L1);
  const float u2 = fmaf(s2, c2, -L2);
  if (TEACHER) return g * exp2_hw(u1) * fmaf(kLn2, u1 - u2, -kl);
  return g * (exp2_hw(u2) - exp2_hw(u1));
}

}  // namespace

// ---------------------------------------------------------------------------
// dK kernel: 4 waves own 128 keys (32 each) of one (b, h) and walk the query
// tiles of 32 rows that see them.  Per step each wave forms S = Q Kᵀ (32
// queries x its 32 keys; key = accumulator column, K in registers), dS in fp32,
// and dK += dSᵀ Q_g with dSᵀ straight from the accumulator registers and Q_g
// from the LDS query tile.  Query tiles are double-buffered in LDS.
// ---------------------------------------------------------------------------
template <typename T, int D1, int D2, bool CAUSAL, bool TEACHER>
__global__ __launch_bounds__(kThreads, 2) void bwd_dk_kernel(const BwdParams p) {
  using M = Mfma<T>;
  using frag = typename M::frag;
  constexpr int KC = M::KC, EPL = M::EPL;
  constexpr int NC1 = D1 / KC, NC2 = D2 / KC;
  constexpr int DG = TEACHER ? D1 : D2;
  constexpr int NCB = DG / 32;
  constexpr int ESZ = sizeof(T);
  constexpr int BQ = kBwdBQ;
  constexpr int PQ1 = D1 * ESZ + kPad, PQ2 = D2 * ESZ + kPad;
  constexpr int PQG = TEACHER ? PQ1 : PQ2;
  constexpr int CPR1 = D1 * ESZ / 16, CPR2 = D2 * ESZ / 16;
  constexpr int NL1 = (BQ * CPR1 + kThreads - 1) / kThreads;  // 16-byte loads per thread
  constexpr int NL2 = (BQ * CPR2 + kThreads - 1) / kThreads;

  __shared__ __attribute__((aligned(16))) char sQ1[2][BQ * PQ1];
  __shared__ __attribute__((aligned(16))) char sQ2[2][BQ * PQ2];
  __shared__ __attribute__((aligned(16))) float sVec[2][4][BQ];  // L1, L2 (base 2), g, KL

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
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

  uint4 pf1[NL1], pf2[NL2];
  float pv = 0.f;
  auto fetch = [&](int64_t q0) {
#pragma unroll
    for (int i = 0; i < NL1; ++i) {
      const int idx = tid + i * kThreads;
      const int row = idx / CPR1, ch = idx % CPR1;
      pf1[i] = make_uint4(0u, 0u, 0u, 0u);
      if (idx < BQ * CPR1 && q0 + row < p.NQ) pf1[i] = ld16(q1p + (q0 + row) * p.sq1.n * ESZ + ch * 16);
    }
#pragma unroll
    for (int i = 0; i < NL2; ++i) {
      const int idx = tid + i * kThreads;
      const int row = idx / CPR2, ch = idx % CPR2;
      pf2[i] = make_uint4(0u, 0u, 0u, 0u);
      if (idx < BQ * CPR2 && q0 + row < p.NQ) pf2[i] = ld16(q2p + (q0 + row) * p.sq2.n * ESZ + ch * 16);
    }
    pv = 0.f;
    if (tid < 4 * BQ) {
      const int which = tid / BQ, row = tid % BQ;
      const int64_t q = q0 + row;
      if (q < p.NQ) {
        const int64_t o = bh * p.NQ + q;
        if (which == 0) pv = p.lse1[o] * kLog2e;
        else if (which == 1) pv = p.lse2[o] * kLog2e;
        else if (which == 2) pv = p.dkl[o];
        else if (TEACHER) pv = p.kl[o];
      }
    }
  };
  auto stash = [&](int st) {
#pragma unroll
    for (int i = 0; i < NL1; ++i) {
      const int idx = tid + i * kThreads;
      if (idx < BQ * CPR1) st16(&sQ1[st][(idx / CPR1) * PQ1 + (idx % CPR1) * 16], pf1[i]);
    }
#pragma unroll
    for (int i = 0; i < NL2; ++i) {
      const int idx = tid + i * kThreads;
      if (idx < BQ * CPR2) st16(&sQ2[st][(idx / CPR2) * PQ2 + (idx % CPR2) * 16], pf2[i]);
    }
    if (tid < 4 * BQ) sVec[st][tid / BQ][tid % BQ] = pv;
  };

  if (nsteps > 0) {
    fetch(qbeg);
    stash(0);
  }
  __syncthreads();
  const float c1 = p.c1, c2 = p.c2;
  const int prow = rperm(col);

  for (int64_t it = 0; it < nsteps; ++it) {
    const int st = (int)(it & 1);
    const int64_t q0 = qbeg + it * BQ;
    if (it + 1 < nsteps) fetch(q0 + BQ);  // next tile in flight during this step

    const bool live = kw0 < p.NK && (!CAUSAL || kw0 <= q0 + BQ - 1 + off);
    if (live) {
      f32x16 s1 = f32x16{}, s2 = f32x16{};
      const char* a1 = &sQ1[st][prow * PQ1 + half * EPL * ESZ];
      const char* a2 = &sQ2[st][prow * PQ2 + half * EPL * ESZ];
#pragma unroll
      for (int c = 0; c < NC1; ++c) s1 = M::run(M::load(a1 + c * KC * ESZ), kf1[c], s1);
#pragma unroll
      for (int c = 0; c < NC2; ++c) s2 = M::run(M::load(a2 + c * KC * ESZ), kf2[c], s2);

      // Per-row values for the 16 rows this lane holds (two runs of 8).
      float vL1[16], vL2[16], vg[16], vkl[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ql = rloc(r, half);
        vL1[r] = sVec[st][0][ql];
        vL2[r] = sVec[st][1][ql];
        vg[r] = sVec[st][2][ql];
        vkl[r] = TEACHER ? sVec[st][3][ql] : 0.f;
      }
      const bool need_mask = (q0 + BQ > p.NQ) || (kw0 + 32 > p.NK) || (CAUSAL && kw0 + 31 > q0 + off);
      f32x16 ds;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = dS_of<TEACHER>(s1[r], s2[r], c1, c2, vL1[r], vL2[r], vg[r], vkl[r]);
        if (need_mask) {
          const int64_t q = q0 + rloc(r, half);
          v = (q < p.NQ && kvalid && (!CAUSAL || key <= q + off)) ? v : 0.f;
        }
        ds[r] = v;
      }

      const char* qg = TEACHER ? &sQ1[st][0] : &sQ2[st][0];
#pragma unroll
      for (int c = 0; c < BQ / KC; ++c) {
        frag a;
        if constexpr (EPL == 1) {
          a = ds[c];
        } else {
#pragma unroll
          for (int e = 0; e < EPL; ++e) a[e] = from_f32<T>(ds[c * EPL + e]);
        }
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          frag bq;
          if constexpr (EPL == 1) {
            bq = *reinterpret_cast<const float*>(qg + rloc(c, half) * PQG + (32 * cb + col) * ESZ);
          } else {
            bq = lds_tr_frag(qg, PQG, c * KC, 32 * cb, lane);
          }
          dk[cb] = M::run(a, bq, dk[cb]);
        }
      }
    }
    if (it + 1 < nsteps) stash(st ^ 1);
    __syncthreads();
  }

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
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_kernel(const BwdParams p) {
  using M = Mfma<T>;
  using frag = typename M::frag;
  constexpr int KC = M::KC, EPL = M::EPL;
  constexpr int NC1 = D1 / KC, NC2 = D2 / KC;
  constexpr int DG = TEACHER ? D1 : D2;
  constexpr int NCB = DG / 32;
  constexpr int ESZ = sizeof(T);
  constexpr int BQ = 128, BK = kDqBK;
  constexpr int PK1 = D1 * ESZ + kPad, PK2 = D2 * ESZ + kPad;
  constexpr int PKG = TEACHER ? PK1 : PK2;
  constexpr int CPR1 = D1 * ESZ / 16, CPR2 = D2 * ESZ / 16;
  constexpr int NL1 = (BK * CPR1 + kThreads - 1) / kThreads;
  constexpr int NL2 = (BK * CPR2 + kThreads - 1) / kThreads;

  __shared__ __attribute__((aligned(16))) char sK1[2][BK * PK1];
  __shared__ __attribute__((aligned(16))) char sK2[2][BK * PK2];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
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

  // Per-row constants: this lane's query row.
  float L1 = 0.f, L2 = 0.f, g = 0.f, klv = 0.f;
  if (qvalid) {
    const int64_t o = bh * p.NQ + qi;
    L1 = p.lse1[o] * kLog2e;
    L2 = p.lse2[o] * kLog2e;
    g = p.dkl[o];
    if (TEACHER) klv = p.kl[o];
  }

  f32x16 dq[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) dq[cb] = f32x16{};

  int64_t kend = p.NK;
  if (CAUSAL) kend = min(kend, (int64_t)(qt + 1) * BQ + off);
  const int64_t nsteps = (kend + BK - 1) / BK;
  const int64_t wave_kmax = CAUSAL ? qw0 + 31 + off : p.NK - 1;

  uint4 pf1[NL1], pf2[NL2];
  auto fetch = [&](int64_t j0) {
#pragma unroll
    for (int i = 0; i < NL1; ++i) {
      const int idx = tid + i * kThreads;
      const int row = idx / CPR1, ch = idx % CPR1;
      pf1[i] = make_uint4(0u, 0u, 0u, 0u);
      if (idx < BK * CPR1 && j0 + row < p.NK) pf1[i] = ld16(k1p + (j0 + row) * p.sk1.n * ESZ + ch * 16);
    }
#pragma unroll
    for (int i = 0; i < NL2; ++i) {
      const int idx = tid + i * kThreads;
      const int row = idx / CPR2, ch = idx % CPR2;
      pf2[i] = make_uint4(0u, 0u, 0u, 0u);
      if (idx < BK * CPR2 && j0 + row < p.NK) pf2[i] = ld16(k2p + (j0 + row) * p.sk2.n * ESZ + ch * 16);
    }
  };
  auto stash = [&](int st) {
#pragma unroll
    for (int i = 0; i < NL1; ++i) {
      const int idx = tid + i * kThreads;
      if (idx < BK * CPR1) st16(&sK1[st][(idx / CPR1) * PK1 + (idx % CPR1) * 16], pf1[i]);
    }
#pragma unroll
    for (int i = 0; i < NL2; ++i) {
      const int idx = tid + i * kThreads;
      if (idx < BK * CPR2) st16(&sK2[st][(idx / CPR2) * PK2 + (idx % CPR2) * 16], pf2[i]);
    }
  };

  if (nsteps > 0) {
    fetch(0);
    stash(0);
  }
  __syncthreads();
  const float c1 = p.c1, c2 = p.c2;
  const int prow = rperm(col);

  for (int64_t it = 0; it < nsteps; ++it) {
    const int st = (int)(it & 1);
    const int64_t j0 = it * BK;
    if (it + 1 < nsteps) fetch(j0 + BK);

    if (j0 <= wave_kmax) {
      const bool need_mask = (j0 + BK > p.NK) || (CAUSAL && j0 + BK - 1 > qw0 + off) || (qw0 + 32 > p.NQ);
      const char* kg = TEACHER ? &sK1[st][0] : &sK2[st][0];
#pragma unroll
      for (int kb = 0; kb < BK / 32; ++kb) {
        f32x16 s1 = f32x16{}, s2 = f32x16{};
        const char* a1 = &sK1[st][(kb * 32 + prow) * PK1 + half * EPL * ESZ];
        const char* a2 = &sK2[st][(kb * 32 + prow) * PK2 + half * EPL * ESZ];
#pragma unroll
        for (int c = 0; c < NC1; ++c) s1 = M::run(M::load(a1 + c * KC * ESZ), qf1[c], s1);
#pragma unroll
        for (int c = 0; c < NC2; ++c) s2 = M::run(M::load(a2 + c * KC * ESZ), qf2[c], s2);
        f32x16 ds;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float v = dS_of<TEACHER>(s1[r], s2[r], c1, c2, L1, L2, g, klv);
          if (need_mask) {
            const int64_t kk = j0 + kb * 32 + rloc(r, half);
            v = (qvalid && kk < p.NK && (!CAUSAL || kk <= qi + off)) ? v : 0.f;
          }
          ds[r] = v;
        }
#pragma unroll
        for (int c = 0; c < 32 / KC; ++c) {
          frag a;
          if constexpr (EPL == 1) {
            a = ds[c];
          } else {
#pragma unroll
            for (int e = 0; e < EPL; ++e) a[e] = from_f32<T>(ds[c * EPL + e]);
          }
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) {
            frag bk;
            if constexpr (EPL == 1) {
              bk = *reinterpret_cast<const float*>(kg + (kb * 32 + rloc(c, half)) * PKG + (32 * cb + col) * ESZ);
            } else {
              bk = lds_tr_frag(kg, PKG, kb * 32 + c * KC, 32 * cb, lane);
            }
            dq[cb] = M::run(a, bk, dq[cb]);
          }
        }
      }
    }
    if (it + 1 < nsteps) stash(st ^ 1);
    __syncthreads();
  }

  // dQ of this wave's rows: accumulator register r holds query qw0 + acc_row(r, half).
  char* const dqp = (char*)p.dq + (b * p.sdq.b + h * p.sdq.h) * ESZ;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t q = qw0 + acc_row(r, half);
      if (q < p.NQ)
        *reinterpret_cast<T*>(dqp + (q * p.sdq.n + 32 * cb + col) * ESZ) = from_f32<T>(dq[cb][r] * p.scale_g);
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
  const int64_t gq = BH * ((p.NQ + 127) / 128);
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
