// Forward kernels of the fused attention-KL primitive for gfx950.
//
// One workgroup = 4 waves = 128 query rows of one (b, h).  It streams the key
// tiles of K1 and K2 through LDS once and, per tile, forms both logit tiles on
// MFMA and updates per-row online statistics (agidaily.cc StreamKL article,
// sections "Online formula" and "Forward: single-pass streaming kernel"):
//
//   m_k  running max of t_k = S_k * log2(e)         (base-2 logits)
//   l_k  running sum of 2^(t_k - m_k)
//   acc  running sum of 2^(t_1 - m_1) * (t_1 - t_2)   (rescaled with m_1 only)
//
// and finishes with KL = ln2 * acc / l1 + LSE2 - LSE1, LSE_k = ln2 (m_k + log2 l_k).
// Only acc, a per-row scalar, needs the correction factor: the logit difference
// is not rescaled by anything, so no d-wide output is rescaled.
//
// Layout on chip.  Each wave computes S^T = K Q^T for its 32 queries: the
// query is the MFMA column (lane % 32), so each lane owns one query row and 16
// keys of every 32-key block.  Row reductions are then in-lane; the two lane
// halves hold disjoint key subsets of the same row and run their own online
// statistics, merged once at the end.  Q fragments stay in registers for the
// whole key loop; K tiles are loaded straight into LDS (direct-to-LDS loads,
// XOR-swizzled rows for conflict-free 16-byte reads), shared by the 4 waves and
// double-buffered: the loads of the next tile are issued before the current
// one is computed.  The online update runs per 32-key block, one block behind
// the MFMAs; a block whose terms stay bounded against the current maxima is
// summed without a new maximum or correction factors (see update below).
//
// Split-K (article section "GPU kernel optimisations"): the same kernel over a
// contiguous key range writes the five per-row partials (m1, l1, m2, l2, acc)
// instead of the final values; reduce_kernel merges them.

#include <type_traits>

#include "skl_device.h"
#include "skl_internal.h"

namespace skl {

// Running maximum of a row before any of its keys has been seen (base-2 logit
// units): finite, so shifts and correction factors never form inf - inf, and
// far enough below any real logit that 2^(t - kNoKey) overflows to +inf.
constexpr float kNoKey = -1e30f;
// Largest block sum kept against a stale running maximum (2^64).
constexpr float kFastCap = 18446744073709551616.0f;
// Update modes of the forward's online statistics (see update in fwd_kernel).
constexpr int kDeferred = 0, kChecked = 1, kFirst = 2;

// Marker written into a row's KL (plain forward) or acc partial (split-K) by
// the main pass when that row needs the fixup pass: a NaN with a payload of
// its own, compared as bits (the file is compiled without NaN semantics).
constexpr uint32_t kRedoMark = 0x7fc0dbadu;

template <typename T, int D1, int D2, bool CAUSAL, bool SPLIT, bool FIXUP>
__global__ __launch_bounds__(kThreads, sizeof(T) == 2 ? 2 : 1) void fwd_kernel(const FwdParams p) {
  using M = Mfma<T>;
  using frag = typename M::frag;
  constexpr int KC = M::KC, EPL = M::EPL;
  constexpr int NC1 = D1 / KC, NC2 = D2 / KC;
  constexpr int ESZ = sizeof(T);
  constexpr int BK = kFwdBK;
  constexpr int RB1 = D1 * ESZ, RB2 = D2 * ESZ;  // bytes per key row
  using T1 = SwzTile<RB1>;
  using T2 = SwzTile<RB2>;
  // The two stages of the ring are separate LDS variables: the compiler can
  // then tell that reads of one stage do not alias the direct-to-LDS loads in
  // flight into the other, and does not wait for those loads before them.
  __shared__ __attribute__((aligned(1024))) char sK1a[BK * RB1], sK1b[BK * RB1];
  __shared__ __attribute__((aligned(1024))) char sK2a[BK * RB2], sK2b[BK * RB2];
  auto sK1 = [&](int st) __attribute__((always_inline)) -> char* { return st ? sK1b : sK1a; };
  auto sK2 = [&](int st) __attribute__((always_inline)) -> char* { return st ? sK2b : sK2a; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int half = lane >> 5, col = lane & 31;

  // Tile decode: logical tile -> (bh, query tile[, split]).
  int64_t t = xcd_remap(blockIdx.x, gridDim.x);
  int split = 0;
  if (SPLIT) {
    split = (int)(t % p.splits);
    t /= p.splits;
  }
  const int64_t bh = t / p.num_qtiles;
  int qt = (int)(t % p.num_qtiles);
  if (CAUSAL) qt = p.num_qtiles - 1 - qt;  // longest rows first
  const int64_t b = bh / p.H, h = bh % p.H;
  const int64_t off = p.NK - p.NQ;

  const int64_t qw0 = (int64_t)qt * kFwdBQ + wave * 32;  // first query of this wave
  const int64_t qi = qw0 + col;                           // this lane's query
  const bool qvalid = qi < p.NQ;
  // Where the main pass left its marker for this row (KL, or the split's acc).
  auto mark_slot = [&]() -> float* {
    if (SPLIT) {
      const int64_t BH = gridDim.x / ((int64_t)p.num_qtiles * p.splits);
      return p.part + 4 * BH * p.splits * p.NQ + (bh * p.splits + split) * p.NQ + qi;
    }
    return p.kl + bh * p.NQ + qi;
  };
  if (FIXUP) {
    // Only tiles with a marked row are recomputed; the others leave at once.
    const bool marked = half == 0 && qvalid && __float_as_uint(*mark_slot()) == kRedoMark;
    if (!__syncthreads_or(marked ? 1 : 0)) return;
  }

  const char* const q1p = (const char*)p.q1 + (b * p.sq1.b + h * p.sq1.h) * ESZ;
  const char* const q2p = (const char*)p.q2 + (b * p.sq2.b + h * p.sq2.h) * ESZ;
  const char* const k1p = (const char*)p.k1 + (b * p.sk1.b + h * p.sk1.h) * ESZ;
  const char* const k2p = (const char*)p.k2 + (b * p.sk2.b + h * p.sk2.h) * ESZ;

  // Q fragments (MFMA B operand: column = query, K slot = head-dim index).
  frag qf1[NC1], qf2[NC2];
#pragma unroll
  for (int c = 0; c < NC1; ++c)
    qf1[c] = qvalid ? M::load(q1p + (qi * p.sq1.n + c * KC + half * EPL) * ESZ) : M::zero();
#pragma unroll
  for (int c = 0; c < NC2; ++c)
    qf2[c] = qvalid ? M::load(q2p + (qi * p.sq2.n + c * KC + half * EPL) * ESZ) : M::zero();

  // Key range of this workgroup and the loop's bounds, all wave-uniform and
  // in 32-bit scalar arithmetic (the host keeps N_Q and N_K below 2^30).
  const int NK = (int)p.NK, offk = (int)off;
  const int qw0s = qt * kFwdBQ + wave * 32;  // first query of this wave
  int kbeg = 0, kend = NK;
  if (CAUSAL) kend = min(kend, (qt + 1) * kFwdBQ + offk);
  if (SPLIT) {
    kbeg = split * p.split_len;
    kend = min(kend, kbeg + p.split_len);
  }
  const int nsteps = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;
  const int wave_kmax = CAUSAL ? qw0s + 31 + offk : NK - 1;  // last key any row of the wave sees
  // A 32-key block starting at jb needs the mask iff it reaches past the last
  // key or (causal) past the diagonal of the wave's first row: jb > mask_after.
  const int mask_after = CAUSAL ? min(NK - 32, qw0s + offk - 31) : NK - 32;

  // Key tiles are loaded straight into a double-buffered LDS ring: the loads
  // of tile i+1 are in flight while tile i is computed; one barrier per tile.
  // A full tile's load instructions take a uniform base (row j0 + 16 k for
  // 256-byte rows, + 32 k for 128-byte rows) in scalar registers plus one
  // loop-invariant lane offset per side: the swizzle repeats every 16 rows,
  // so all of a wave's instructions share that offset.  The ragged last tile
  // takes the clamping loader.
  const int64_t rs1 = p.sk1.n * ESZ, rs2 = p.sk2.n * ESZ;
  constexpr int RPI1 = 1024 / RB1, RPI2 = 1024 / RB2;  // rows per load instruction
  const int r01 = wave * RPI1 + lane / T1::CPR, r02 = wave * RPI2 + lane / T2::CPR;
  const unsigned lo1 = (unsigned)(r01 * (int)rs1 + (((lane % T1::CPR) ^ T1::swz(r01)) * 16));
  const unsigned lo2 = (unsigned)(r02 * (int)rs2 + (((lane % T2::CPR) ^ T2::swz(r02)) * 16));
  auto fetch = [&](int st, int j0) {
    if (j0 + BK <= NK) {
      // Fresh copies of the lane offsets here, so that they are not hoisted
      // as 64-bit values (which loses the scalar-base form of the loads).
      unsigned o1 = lo1, o2 = lo2;
      asm volatile("" : "+v"(o1), "+v"(o2));
#pragma unroll
      for (int k = 0; k < BK / RPI1 / 4; ++k)
        global_load_lds16(uniform_ptr(k1p + (int64_t)(j0 + 4 * k * RPI1) * rs1) + o1, sK1(st) + (wave + 4 * k) * 1024);
#pragma unroll
      for (int k = 0; k < BK / RPI2 / 4; ++k)
        global_load_lds16(uniform_ptr(k2p + (int64_t)(j0 + 4 * k * RPI2) * rs2) + o2, sK2(st) + (wave + 4 * k) * 1024);
    } else {
      tile_load_async<BK, RB1>(sK1(st), k1p, rs1, j0, NK, wave, lane);
      tile_load_async<BK, RB2>(sK2(st), k2p, rs2, j0, NK, wave, lane);
    }
  };

  const float c1 = p.c1, c2 = p.c2;
  // Running maxima in base-2 units start at the finite kNoKey ("no key seen"),
  // so that every shift and correction factor below is finite.
  float m1 = kNoKey, m2 = kNoKey, l1 = 0.f, l2 = 0.f, acc = 0.f;
  bool over = false;  // a kept-maximum block exceeded the cap (deferred check)

  // Per-lane byte offsets of the A fragments inside a 32-row block: the
  // swizzle repeats every 16 rows, so block kb of stage st is at the constant
  // st * BK * RB + kb * 32 * RB from these (an immediate of the LDS read).
  int aoff1[NC1], aoff2[NC2];
#pragma unroll
  for (int c = 0; c < NC1; ++c) aoff1[c] = T1::off(col, (c * KC + half * EPL) * ESZ);
#pragma unroll
  for (int c = 0; c < NC2; ++c) aoff2[c] = T2::off(col, (c * KC + half * EPL) * ESZ);

  static_assert(BK == 64, "the block pipeline below assumes two 32-key blocks per tile");

  // Logits of 32-key block kb of ring stage ST: all A fragments are read
  // first, then the two MFMA chains are interleaved.
  auto logits = [&](auto stc, int kb, f32x16& s1, f32x16& s2) {
    constexpr int st = decltype(stc)::value;
    frag ka1[NC1], ka2[NC2];
#pragma unroll
    for (int c = 0; c < NC1; ++c) ka1[c] = M::load(&sK1(st)[kb * 32 * RB1 + aoff1[c]]);
#pragma unroll
    for (int c = 0; c < NC2; ++c) ka2[c] = M::load(&sK2(st)[kb * 32 * RB2 + aoff2[c]]);
    s1 = f32x16{};
    s2 = f32x16{};
    // Raised wave priority while the MFMAs issue: the other wave of the SIMD,
    // in its VALU phase, then fills the gaps instead of competing for issue,
    // which keeps the two waves out of phase.
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int c = 0; c < (NC1 > NC2 ? NC1 : NC2); ++c) {
      if (c < NC1) s1 = M::run(ka1[c], qf1[c], s1);
      if (c < NC2) s2 = M::run(ka2[c], qf2[c], s2);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // Online update of the row statistics with one block whose first key is jb.
  //
  // Most blocks keep the running maxima: the block is summed against the
  // current (m1, m2), and that result is valid whenever both of its sums stay
  // at or below kFastCap = 2^64, which bounds every term by 2^64 (far from
  // fp32 overflow even after summing 2^20 blocks).  A stale maximum only makes
  // the terms larger, never smaller, so nothing underflows that the exact
  // update would keep; the sums are the same quantities in another base-2
  // unit.  The exact update of the online formula (new block maximum,
  // correction factors, rescale) is needed only when a block exceeds the cap
  // or no key has been seen yet.  Modes:
  //   kFirst     the first block of the key range: always the exact update
  //              (it sets the maxima from the block's own logits);
  //   kDeferred  every later block on the main pass: the kept-maximum sums
  //              are committed without a branch and a block over the cap only
  //              sets `over`; the workgroup then repeats its key range in
  //              kChecked mode (rare: logits rising by more than ~64 bits of
  //              range after the first block);
  //   kChecked   per block, the exact update only where the cap is exceeded.
  auto update = [&](auto modec, f32x16& s1, f32x16& s2, int jb) __attribute__((always_inline)) {
    constexpr int mode = decltype(modec)::value;
    const bool need_mask = jb > mask_after;
    if (need_mask) {
      // Key jb + ro is visible iff ro < NK - jb and (causal) ro <= qi + off - jb.
      const int klim = NK - jb, cmax = (int)qi + offk - jb;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ro = acc_row(r, half);
        if (!(ro < klim && (!CAUSAL || ro <= cmax))) {
          s1[r] = neg_inf();
          s2[r] = neg_inf();
        }
      }
    }

    // Block sums against the shifts (sh1, sh2): sum_k = sum 2^(t_k - sh_k) and
    // accd = sum 2^(t1 - sh1) * (u1 - u2) with u_k = t_k - sh_k.  They run as 4
    // independent chains (with two waves per SIMD a single dependent chain of 16
    // would leave the VALU waiting on its own latency), each started by its
    // first term rather than by adding it to zero.
    auto block_sums = [&](float sh1, float sh2, float& sum1, float& sum2, float& accd)
        __attribute__((always_inline)) {
      float ps1[4], ps2[4], pa[4];
      auto term = [&](int r, float u1, float u2, float d) __attribute__((always_inline)) {
        const float e1 = exp2_hw(u1), e2 = exp2_hw(u2);
        if (r < 4) {
          ps1[r] = e1;
          ps2[r] = e2;
          pa[r] = e1 * d;
        } else {
          ps1[r & 3] += e1;
          ps2[r & 3] += e2;
          pa[r & 3] = fmaf(e1, d, pa[r & 3]);
        }
      };
      if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float u1 = fmaf(s1[r], c1, -sh1), u2 = fmaf(s2[r], c2, -sh2);
          term(r, u1, u2, (s1[r] == neg_inf()) ? 0.f : (u1 - u2));
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float u1 = fmaf(s1[r], c1, -sh1), u2 = fmaf(s2[r], c2, -sh2);
          term(r, u1, u2, u1 - u2);
        }
      }
      sum1 = (ps1[0] + ps1[1]) + (ps1[2] + ps1[3]);
      sum2 = (ps2[0] + ps2[1]) + (ps2[2] + ps2[3]);
      accd = (pa[0] + pa[1]) + (pa[2] + pa[3]);
    };

    // Exact update: block maxima of the raw logits as a tree of 3-input
    // maxima, scaled afterwards (the scales are positive) and joined with the
    // running maxima (a lane whose keys are all masked keeps its maxima).
    auto exact = [&]() __attribute__((always_inline)) {
      auto max3 = [](float a, float b, float c) __attribute__((always_inline)) { return fmaxf(fmaxf(a, b), c); };
      auto tree = [&](const f32x16& v) __attribute__((always_inline)) {
        const float b0 = max3(max3(v[0], v[1], v[2]), max3(v[3], v[4], v[5]), max3(v[6], v[7], v[8]));
        const float b1 = max3(max3(v[9], v[10], v[11]), max3(v[12], v[13], v[14]), v[15]);
        return fmaxf(b0, b1);
      };
      const float m1n = fmaxf(tree(s1) * c1, m1), m2n = fmaxf(tree(s2) * c2, m2);
      const float a1f = exp2_hw(m1 - m1n), a2f = exp2_hw(m2 - m2n);
      float sum1, sum2, accd;
      block_sums(m1n, m2n, sum1, sum2, accd);
      l1 = fmaf(l1, a1f, sum1);
      l2 = fmaf(l2, a2f, sum2);
      acc = fmaf(acc, a1f, fmaf(m1n - m2n, sum1, accd));
      m1 = m1n;
      m2 = m2n;
    };

    if constexpr (mode == kFirst) {
      exact();
    } else {
      float sum1, sum2, accd;
      block_sums(m1, m2, sum1, sum2, accd);
      const bool fits = sum1 <= kFastCap && sum2 <= kFastCap;
      // t1 - t2 = (u1 - u2) + (m1 - m2): the per-row part is added once per block.
      const float nl1 = l1 + sum1, nl2 = l2 + sum2, nacc = acc + fmaf(m1 - m2, sum1, accd);
      if constexpr (mode == kDeferred) {
        over |= !fits;
        l1 = nl1;
        l2 = nl2;
        acc = nacc;
      } else {
        if (fits) {
          l1 = nl1;
          l2 = nl2;
          acc = nacc;
        } else {
          exact();
        }
      }
    }
  };

  // Block-level software pipeline: the MFMAs of the next 32-key block are
  // issued before the online update of the current one (across the tile
  // barrier too), so each wave keeps matrix work in flight while its VALU
  // runs the softmax.  Blocks past the wave's last visible key are skipped.
  // The first step is peeled so that only its first block takes kFirst.  The
  // main pass commits later blocks in kDeferred mode and marks the rows that
  // went over the cap; the fixup pass (FIXUP) repeats such tiles in kChecked
  // mode.
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using First = std::integral_constant<int, kFirst>;
  using Later = std::integral_constant<int, FIXUP ? kChecked : kDeferred>;
  f32x16 sa1, sa2, sb1, sb2;  // block 0 / block 1 of the current tile
  auto step = [&](auto stc, int it, auto mode0) {
    constexpr int st = decltype(stc)::value;
    const int j0 = kbeg + it * BK;
    if (it + 1 < nsteps) fetch(st ^ 1, j0 + BK);
    const bool live0 = j0 <= wave_kmax, live1 = j0 + 32 <= wave_kmax;
    if (live1) logits(stc, 1, sb1, sb2);
    if (live0) update(mode0, sa1, sa2, j0);
    wait_vm();
    __syncthreads();
    if (it + 1 < nsteps && j0 + BK <= wave_kmax) logits(std::integral_constant<int, st ^ 1>{}, 0, sa1, sa2);
    if (live1) update(Later{}, sb1, sb2, j0 + 32);
  };
  if (nsteps > 0) fetch(0, kbeg);
  wait_vm();
  __syncthreads();
  if (nsteps > 0) {
    if (kbeg <= wave_kmax) logits(I0{}, 0, sa1, sa2);
    step(I0{}, 0, First{});
  }
  for (int it = 1; it < nsteps; it += 2) {
    step(I1{}, it, Later{});
    if (it + 1 < nsteps) step(I0{}, it + 1, Later{});
  }
  const bool redo = over || __shfl_xor(over ? 1 : 0, 32) != 0;

  // Merge the two lane halves (disjoint key subsets of the same row).
  const float om1 = __shfl_xor(m1, 32), ol1 = __shfl_xor(l1, 32);
  const float om2 = __shfl_xor(m2, 32), ol2 = __shfl_xor(l2, 32);
  const float oacc = __shfl_xor(acc, 32);
  const float M1 = fmaxf(m1, om1), M2 = fmaxf(m2, om2);
  const float wa1 = exp2_hw(m1 - M1), wb1 = exp2_hw(om1 - M1);
  const float wa2 = exp2_hw(m2 - M2), wb2 = exp2_hw(om2 - M2);
  const float L1 = l1 * wa1 + ol1 * wb1;
  const float L2 = l2 * wa2 + ol2 * wb2;
  const float ACC = acc * wa1 + oacc * wb1;

  if (half == 0 && qvalid) {
    if (SPLIT) {
      const int64_t BH = gridDim.x / ((int64_t)p.num_qtiles * p.splits);
      const int64_t stride_f = BH * p.splits * p.NQ;
      float* dst = p.part + (bh * p.splits + split) * p.NQ + qi;
      // A split in which the row saw no key writes (-inf, 0, -inf, 0, 0).
      dst[0] = (L1 > 0.f) ? M1 : neg_inf();
      dst[stride_f] = L1;
      dst[2 * stride_f] = (L2 > 0.f) ? M2 : neg_inf();
      dst[3 * stride_f] = L2;
      dst[4 * stride_f] = redo ? __uint_as_float(kRedoMark) : ACC;
    } else {
      const float lg1 = log2f(L1), lg2 = log2f(L2);
      const int64_t o = bh * p.NQ + qi;
      p.lse1[o] = kLn2 * (M1 + lg1);
      p.lse2[o] = kLn2 * (M2 + lg2);
      p.kl[o] = redo ? __uint_as_float(kRedoMark) : kLn2 * (ACC / L1 + (M2 - M1) + (lg2 - lg1));
    }
  }
}

// Merge split-K partials: one thread per row (grid-stride, so any row count
// fits one launch).
__global__ __launch_bounds__(256) void reduce_kernel(const ReduceParams p) {
  for (int64_t row = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; row < p.rows;
       row += (int64_t)gridDim.x * blockDim.x) {
    const int64_t bh = row / p.NQ, i = row % p.NQ;
    const int64_t stride_f = p.rows * p.splits;
    const float* src = p.part + bh * p.splits * p.NQ + i;
    float M1 = neg_inf(), M2 = neg_inf();
    for (int s = 0; s < p.splits; ++s) {
      M1 = fmaxf(M1, src[s * p.NQ]);
      M2 = fmaxf(M2, src[2 * stride_f + s * p.NQ]);
    }
    const float M1u = (M1 == neg_inf()) ? 0.f : M1;
    const float M2u = (M2 == neg_inf()) ? 0.f : M2;
    float L1 = 0.f, L2 = 0.f, ACC = 0.f;
    for (int s = 0; s < p.splits; ++s) {
      const float w1 = exp2_hw(src[s * p.NQ] - M1u);
      const float w2 = exp2_hw(src[2 * stride_f + s * p.NQ] - M2u);
      L1 = fmaf(src[stride_f + s * p.NQ], w1, L1);
      ACC = fmaf(src[4 * stride_f + s * p.NQ], w1, ACC);
      L2 = fmaf(src[3 * stride_f + s * p.NQ], w2, L2);
    }
    const float lg1 = log2f(L1), lg2 = log2f(L2);
    p.lse1[row] = kLn2 * (M1 + lg1);
    p.lse2[row] = kLn2 * (M2 + lg2);
    p.kl[row] = kLn2 * (ACC / L1 + (M2 - M1) + (lg2 - lg1));
  }
}

namespace {

// The main pass, then the fixup pass over the same tiles (most of its
// workgroups find no marked row and leave at once).  `between` runs after the
// main pass's launch (profiling events).
template <typename T, int D1, int D2, bool C, bool S>
hipError_t run_fwd(const FwdParams& p, int64_t BH, hipStream_t s, void (*between)(hipStream_t)) {
  const int64_t grid = BH * p.num_qtiles * (S ? p.splits : 1);
  hipLaunchKernelGGL((fwd_kernel<T, D1, D2, C, S, false>), dim3((unsigned)grid), dim3(kThreads), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (between) between(s);
  hipLaunchKernelGGL((fwd_kernel<T, D1, D2, C, S, true>), dim3((unsigned)grid), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

template <typename T, int D1, int D2>
hipError_t fwd_dims(const FwdParams& p, bool causal, bool split, int64_t BH, hipStream_t s,
                    void (*bw)(hipStream_t)) {
  if (causal)
    return split ? run_fwd<T, D1, D2, true, true>(p, BH, s, bw) : run_fwd<T, D1, D2, true, false>(p, BH, s, bw);
  return split ? run_fwd<T, D1, D2, false, true>(p, BH, s, bw) : run_fwd<T, D1, D2, false, false>(p, BH, s, bw);
}

template <typename T>
hipError_t fwd_type(const FwdParams& p, int d1, int d2, bool causal, bool split, int64_t BH, hipStream_t s,
                    void (*bw)(hipStream_t)) {
  if (d1 == 128 && d2 == 128) return fwd_dims<T, 128, 128>(p, causal, split, BH, s, bw);
  if (d1 == 128 && d2 == 64) return fwd_dims<T, 128, 64>(p, causal, split, BH, s, bw);
  if (d1 == 64 && d2 == 128) return fwd_dims<T, 64, 128>(p, causal, split, BH, s, bw);
  if (d1 == 64 && d2 == 64) return fwd_dims<T, 64, 64>(p, causal, split, BH, s, bw);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_forward(const FwdParams& p, int dtype, int d1, int d2, bool causal, bool split,
                          int64_t BH, hipStream_t s, void (*between)(hipStream_t)) {
  if (dtype == 0) return fwd_type<bf16>(p, d1, d2, causal, split, BH, s, between);
  return fwd_type<float>(p, d1, d2, causal, split, BH, s, between);
}

hipError_t launch_reduce(const ReduceParams& p, hipStream_t s) {
  int64_t blocks = (p.rows + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace skl
