// Fused backward kernel of the attention-KL primitive for gfx950 (the
// SKL_BWD_FUSED_ATOMIC algorithm; bwd_split.hip holds the default one).
//
// Recompute-based (agidaily.cc StreamKL article, section "Backward:
// recompute-based tile-by-tile gradients"): P1 = 2^(t1 - LSE1*log2e) and
// P2 = 2^(t2 - LSE2*log2e) are rebuilt tile by tile from the saved LSEs, for
// the two gradient settings
//   student (optimise P2):  dS2 = g (P2 - P1)
//   teacher (optimise P1):  dS1 = g P1 (r - KL),  r = ln2 ((t1 - L1) - (t2 - L2))
// where r is the log-ratio formed from logits, so an underflowed P1 gives an
// exact 0 instead of 0 * (-inf).
//
// Fusion (article section "GPU kernel optimisations", fused backward): one
// workgroup owns 128 keys (4 waves x 32) and walks the query tiles (32 rows)
// that can see them, so every (query tile, key tile) pair is visited once.
// dK of its keys accumulates in MFMA registers; dQ of each query tile is
// reduced over the workgroup's 128 keys on chip and added to an fp32
// workspace with one atomic per element; a convert kernel applies the scale
// and the output dtype afterwards.
//
// MFMA orientation.  Each wave computes S = Q K^T for 32 queries x its 32
// keys; the key is the accumulator column (lane % 32).  The query rows of the
// A operand are loaded in a permuted order so that accumulator register r of
// lane half h holds query rloc(r, h) = 16 (r / 8) + 8 h + r % 8: the registers
// then are directly the A operand of dK += dS^T Q (contraction over queries,
// 8 consecutive queries per lane).  dQ = dS K contracts over keys, so dS makes
// one trip through LDS (the only transpose), and K is kept transposed in
// registers as the B operand.

#include "skl_device.h"
#include "skl_internal.h"

namespace skl {


template <typename T, int D1, int D2, bool CAUSAL, bool TEACHER>
__global__ __launch_bounds__(kThreads, sizeof(T) == 2 ? 2 : 1) void bwd_fused_kernel(const BwdParams p) {
  using M = Mfma<T>;
  using frag = typename M::frag;
  constexpr int KC = M::KC, EPL = M::EPL;
  constexpr int NC1 = D1 / KC, NC2 = D2 / KC;
  constexpr int DG = TEACHER ? D1 : D2;      // head dim of the optimised side
  constexpr int NCB = DG / 32;               // 32-wide column blocks of dQ / dK
  constexpr int KSPLIT = 4 / NCB;            // waves sharing one dQ block
  constexpr int KPART = kBwdBK / KSPLIT;     // keys per dQ partial
  constexpr int ESZ = sizeof(T);
  constexpr int PQ1 = D1 * ESZ + 16;         // LDS pitches in bytes
  constexpr int PQ2 = D2 * ESZ + 16;
  constexpr int PQT = kBwdBQ * ESZ + 16;
  constexpr int PDS = kBwdBK * ESZ + 16;
  constexpr int CPR1 = D1 * ESZ / 16, CPR2 = D2 * ESZ / 16;
  constexpr int EPC = 16 / ESZ;              // elements per 16-byte chunk
  static_assert(NCB * KSPLIT == 4, "dQ blocks must cover the 4 waves");

  __shared__ __attribute__((aligned(16))) char sQ1[kBwdBQ * PQ1];
  __shared__ __attribute__((aligned(16))) char sQ2[kBwdBQ * PQ2];
  __shared__ __attribute__((aligned(16))) char sQT[DG * PQT];      // optimised-side Q, transposed
  __shared__ __attribute__((aligned(16))) char sDS[kBwdBQ * PDS];  // dS, [query][key]
  __shared__ __attribute__((aligned(16))) float sVec[4][kBwdBQ];   // L1, L2 (base 2), g, KL
  __shared__ __attribute__((aligned(16))) float sRed[KSPLIT > 1 ? NCB * 16 * 64 : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5, col = lane & 31;

  const int64_t t = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t bh = t / p.num_ktiles;
  const int kt = (int)(t % p.num_ktiles);
  const int64_t b = bh / p.H, h = bh % p.H;
  const int64_t off = p.NK - p.NQ;
  const int64_t kt0 = (int64_t)kt * kBwdBK;
  const int64_t kw0 = kt0 + 32 * wave;  // this wave's first key
  const int64_t key = kw0 + col;        // this lane's key (accumulator column)
  const bool kvalid = key < p.NK;

  const char* const q1p = (const char*)p.q1 + (b * p.sq1.b + h * p.sq1.h) * ESZ;
  const char* const q2p = (const char*)p.q2 + (b * p.sq2.b + h * p.sq2.h) * ESZ;
  const char* const k1p = (const char*)p.k1 + (b * p.sk1.b + h * p.sk1.h) * ESZ;
  const char* const k2p = (const char*)p.k2 + (b * p.sk2.b + h * p.sk2.h) * ESZ;
  const char* const kgp = TEACHER ? k1p : k2p;
  const int64_t kg_n = TEACHER ? p.sk1.n : p.sk2.n;

  // K fragments as the B operand of S = Q K^T (column = key, K slot = head dim).
  frag kf1[NC1], kf2[NC2];
#pragma unroll
  for (int c = 0; c < NC1; ++c)
    kf1[c] = kvalid ? M::load(k1p + (key * p.sk1.n + c * KC + half * EPL) * ESZ) : M::zero();
#pragma unroll
  for (int c = 0; c < NC2; ++c)
    kf2[c] = kvalid ? M::load(k2p + (key * p.sk2.n + c * KC + half * EPL) * ESZ) : M::zero();

  // Optimised-side K, transposed, as the B operand of dQ = dS K
  // (column = head-dim index, K slot = key).  Loaded once per workgroup.
  const int cb_q = wave % NCB, kp_q = wave / NCB;  // this wave's dQ block / key part
  frag kgt[KPART / KC];
#pragma unroll
  for (int c = 0; c < KPART / KC; ++c) {
    if constexpr (EPL == 1) {
      const int64_t kk = kt0 + kp_q * KPART + c * KC + half;
      kgt[c] = kk < p.NK ? *reinterpret_cast<const float*>(kgp + (kk * kg_n + 32 * cb_q + col) * ESZ) : 0.f;
    } else {
      frag v;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const int64_t kk = kt0 + kp_q * KPART + c * KC + half * EPL + e;
        v[e] = kk < p.NK ? *reinterpret_cast<const T*>(kgp + (kk * kg_n + 32 * cb_q + col) * ESZ) : T(0.f);
      }
      kgt[c] = v;
    }
  }

  f32x16 dk[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) dk[cb] = f32x16{};

  const float c1 = p.c1, c2 = p.c2;
  const int prow = rperm(col);
  int64_t qbeg = 0;
  if (CAUSAL) qbeg = max((int64_t)0, kt0 - off) / kBwdBQ * kBwdBQ;

  for (int64_t q0 = qbeg; q0 < p.NQ; q0 += kBwdBQ) {
    __syncthreads();  // LDS of the previous step fully consumed
    // Stage Q1, Q2 rows (and the optimised side transposed) plus per-row vectors.
    for (int idx = tid; idx < kBwdBQ * CPR1; idx += kThreads) {
      const int row = idx / CPR1, ch = idx % CPR1;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (q0 + row < p.NQ) v = ld16(q1p + (q0 + row) * p.sq1.n * ESZ + ch * 16);
      st16(sQ1 + row * PQ1 + ch * 16, v);
      if (TEACHER) {
        const T* e = reinterpret_cast<const T*>(&v);
#pragma unroll
        for (int x = 0; x < EPC; ++x) *reinterpret_cast<T*>(sQT + (ch * EPC + x) * PQT + row * ESZ) = e[x];
      }
    }
    for (int idx = tid; idx < kBwdBQ * CPR2; idx += kThreads) {
      const int row = idx / CPR2, ch = idx % CPR2;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (q0 + row < p.NQ) v = ld16(q2p + (q0 + row) * p.sq2.n * ESZ + ch * 16);
      st16(sQ2 + row * PQ2 + ch * 16, v);
      if (!TEACHER) {
        const T* e = reinterpret_cast<const T*>(&v);
#pragma unroll
        for (int x = 0; x < EPC; ++x) *reinterpret_cast<T*>(sQT + (ch * EPC + x) * PQT + row * ESZ) = e[x];
      }
    }
    if (tid < 4 * kBwdBQ) {
      const int which = tid / kBwdBQ, row = tid % kBwdBQ;
      const int64_t q = q0 + row;
      float v = 0.f;
      if (q < p.NQ) {
        const int64_t o = bh * p.NQ + q;
        if (which == 0) v = p.lse1[o] * kLog2e;
        else if (which == 1) v = p.lse2[o] * kLog2e;
        else if (which == 2) v = p.dkl[o];
        else if (TEACHER) v = p.kl[o];
      }
      sVec[which][row] = v;
    }
    __syncthreads();

    // dS for (32 queries) x (this wave's 32 keys), in accumulator layout.
    f32x16 ds = f32x16{};
    const bool wave_live = kw0 < p.NK && (!CAUSAL || kw0 <= q0 + kBwdBQ - 1 + off);
    if (wave_live) {
      f32x16 s1 = f32x16{}, s2 = f32x16{};
      const char* a1 = sQ1 + prow * PQ1 + half * EPL * ESZ;
      const char* a2 = sQ2 + prow * PQ2 + half * EPL * ESZ;
#pragma unroll
      for (int c = 0; c < NC1; ++c) s1 = M::run(M::load(a1 + c * KC * ESZ), kf1[c], s1);
#pragma unroll
      for (int c = 0; c < NC2; ++c) s2 = M::run(M::load(a2 + c * KC * ESZ), kf2[c], s2);

      const bool need_mask = (q0 + kBwdBQ > p.NQ) || (kw0 + 32 > p.NK) ||
                             (CAUSAL && kw0 + 31 > q0 + off);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ql = rloc(r, half);
        const float u1 = fmaf(s1[r], c1, -sVec[0][ql]);
        const float u2 = fmaf(s2[r], c2, -sVec[1][ql]);
        const float g = sVec[2][ql];
        float v;
        if (TEACHER) {
          v = g * exp2_hw(u1) * fmaf(kLn2, u1 - u2, -sVec[3][ql]);
        } else {
          v = g * (exp2_hw(u2) - exp2_hw(u1));
        }
        if (need_mask) {
          const int64_t q = q0 + ql;
          const bool ok = q < p.NQ && kvalid && (!CAUSAL || key <= q + off);
          v = ok ? v : 0.f;
        }
        ds[r] = v;
      }

      // dK += dS^T Q  (A = dS^T straight from the accumulator registers).
#pragma unroll
      for (int c = 0; c < kBwdBQ / KC; ++c) {
        frag a;
        if constexpr (EPL == 1) {
          a = ds[c];
        } else {
#pragma unroll
          for (int e = 0; e < EPL; ++e) a[e] = from_f32<T>(ds[c * EPL + e]);
        }
        const int qs = (EPL == 1) ? rloc(c, half) : c * KC + half * EPL;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          const frag bq = M::load(sQT + (32 * cb + col) * PQT + qs * ESZ);
          dk[cb] = M::run(a, bq, dk[cb]);
        }
      }
    }
    // dS -> LDS as [query][key] for the dQ contraction over keys.
#pragma unroll
    for (int r = 0; r < 16; ++r)
      *reinterpret_cast<T*>(sDS + rloc(r, half) * PDS + (32 * wave + col) * ESZ) = from_f32<T>(ds[r]);
    __syncthreads();

    // dQ block (32 queries x 32 columns) over this wave's key part.
    f32x16 dq = f32x16{};
    const char* ad = sDS + col * PDS + (kp_q * KPART + half * EPL) * ESZ;
#pragma unroll
    for (int c = 0; c < KPART / KC; ++c) dq = M::run(M::load(ad + c * KC * ESZ), kgt[c], dq);
    if constexpr (KSPLIT > 1) {
      float* red = sRed + cb_q * 16 * 64;
      if (kp_q == 1) {
#pragma unroll
        for (int r = 0; r < 16; ++r) red[r * 64 + lane] = dq[r];
      }
      __syncthreads();
      if (kp_q == 0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) dq[r] += red[r * 64 + lane];
      }
    }
    if (kp_q == 0) {
      float* wrow = p.ws + (bh * p.NQ + q0) * DG + 32 * cb_q + col;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qr = acc_row(r, half);
        if (q0 + qr < p.NQ) unsafeAtomicAdd(wrow + (int64_t)qr * DG, dq[r]);
      }
    }
  }

  // dK of this wave's keys: accumulator register r holds key kw0 + acc_row(r, half).
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

__global__ __launch_bounds__(256) void zero_kernel(float4* __restrict__ ws, int64_t n4) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x)
    ws[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// Zeros into a strided [B, H, N, d] tensor with a contiguous d axis and
// 16-byte aligned rows: the key gradient of a backward call with no query
// rows, where no kernel above runs.
__global__ __launch_bounds__(256) void zero_rows_kernel(char* __restrict__ base, const Strides st, int64_t H,
                                                        int64_t N, int64_t rows, int chunks, int esz) {
  const int64_t n = rows * chunks;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = i / chunks;
    const int64_t bh = row / N, r = row % N;
    const int64_t b = bh / H, h = bh % H;
    float4* dst = reinterpret_cast<float4*>(base + (b * st.b + h * st.h + r * st.n) * esz) + (i % chunks);
    *dst = make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

// ws fp32 [B*H][NQ][dg] -> dq (input dtype, caller strides) times scale.
template <typename T>
__global__ __launch_bounds__(256) void convert_kernel(const ConvertParams p) {
  constexpr int V = 4;
  const int64_t per_row = p.dg / V;
  const int64_t n = p.rows * per_row;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = i / per_row;
    const int d0 = (int)(i % per_row) * V;
    const int64_t bh = row / p.NQ, q = row % p.NQ;
    const int64_t b = bh / p.H, h = bh % p.H;
    float4 v = reinterpret_cast<const float4*>(p.ws)[i];
    for (int sp = 1; sp < p.splits; ++sp) {
      const float4 u = reinterpret_cast<const float4*>(p.ws + sp * p.split_stride)[i];
      v.x += u.x;
      v.y += u.y;
      v.z += u.z;
      v.w += u.w;
    }
    T* dst = reinterpret_cast<T*>(p.dq) + b * p.sdq.b + h * p.sdq.h + q * p.sdq.n + d0;
    dst[0] = from_f32<T>(v.x * p.scale);
    dst[1] = from_f32<T>(v.y * p.scale);
    dst[2] = from_f32<T>(v.z * p.scale);
    dst[3] = from_f32<T>(v.w * p.scale);
  }
}

namespace {

template <typename T, int D1, int D2, bool C, bool TCH>
hipError_t run_bwd(const BwdParams& p, int64_t BH, hipStream_t s) {
  const int64_t grid = BH * p.num_ktiles;
  hipLaunchKernelGGL((bwd_fused_kernel<T, D1, D2, C, TCH>), dim3((unsigned)grid), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

template <typename T, int D1, int D2>
hipError_t bwd_dims(const BwdParams& p, bool causal, bool teacher, int64_t BH, hipStream_t s) {
  if (causal) return teacher ? run_bwd<T, D1, D2, true, true>(p, BH, s) : run_bwd<T, D1, D2, true, false>(p, BH, s);
  return teacher ? run_bwd<T, D1, D2, false, true>(p, BH, s) : run_bwd<T, D1, D2, false, false>(p, BH, s);
}

template <typename T>
hipError_t bwd_type(const BwdParams& p, int d1, int d2, bool causal, bool teacher, int64_t BH, hipStream_t s) {
  if (d1 == 128 && d2 == 128) return bwd_dims<T, 128, 128>(p, causal, teacher, BH, s);
  if (d1 == 128 && d2 == 64) return bwd_dims<T, 128, 64>(p, causal, teacher, BH, s);
  if (d1 == 64 && d2 == 128) return bwd_dims<T, 64, 128>(p, causal, teacher, BH, s);
  if (d1 == 64 && d2 == 64) return bwd_dims<T, 64, 64>(p, causal, teacher, BH, s);
  return hipErrorInvalidValue;
}

int64_t grid_for(int64_t n, int64_t per_block) {
  const int64_t g = (n + per_block - 1) / per_block;
  return g < 1 ? 1 : (g > 65536 ? 65536 : g);
}

}  // namespace

hipError_t launch_backward_fused(const BwdParams& p, int dtype, int d1, int d2, bool causal, bool teacher,
                                 int64_t BH, hipStream_t s) {
  if (dtype == 0) return bwd_type<bf16>(p, d1, d2, causal, teacher, BH, s);
  return bwd_type<float>(p, d1, d2, causal, teacher, BH, s);
}

hipError_t launch_zero(float* ws, int64_t count, hipStream_t s) {
  const int64_t n4 = count / 4;  // count is a multiple of 64 (head dims 64 / 128)
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)grid_for(n4, 256)), dim3(256), 0, s,
                     reinterpret_cast<float4*>(ws), n4);
  return hipGetLastError();
}

hipError_t launch_zero_rows(void* dst, const Strides& st, int64_t B, int64_t H, int64_t N, int d, int dtype,
                            hipStream_t s) {
  const int esz = dtype == 0 ? 2 : 4;
  const int chunks = d * esz / 16;  // 16-byte pieces per row (head dims 64 / 128)
  const int64_t rows = B * H * N;
  hipLaunchKernelGGL(zero_rows_kernel, dim3((unsigned)grid_for(rows * chunks, 256)), dim3(256), 0, s,
                     static_cast<char*>(dst), st, H, N, rows, chunks, esz);
  return hipGetLastError();
}

hipError_t launch_convert(const ConvertParams& p, int dtype, hipStream_t s) {
  const int64_t n = p.rows * (p.dg / 4);
  const dim3 grid((unsigned)grid_for(n, 256));
  if (dtype == 0)
    hipLaunchKernelGGL(convert_kernel<bf16>, grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(convert_kernel<float>, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace skl
