// Device-side helpers shared by the gfx950 kernels: element types, MFMA
// wrappers, fragment loads and base-2 exponentials.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace skl {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// v_exp_f32: 2^x on the transcendental unit (no libm wrapper).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// One 32x32 MFMA step, D = A*B + C with fp32 accumulation.
//  * bf16: v_mfma_f32_32x32x16_bf16, K = 16, each lane holds 8 K-values.
//  * fp32: v_mfma_f32_32x32x2_f32,   K = 2,  each lane holds 1 K-value.
// Operand layout (both types): lane l supplies A[i = l % 32][kslot(l / 32)]
// and B[kslot(l / 32)][j = l % 32]; the accumulator register r of lane l is
// D[8 * (r / 4) + 4 * (l / 32) + r % 4][l % 32].  Which K index each
// (lane half, element) slot carries does not matter as long as A and B agree.
template <typename T>
struct Mfma;

template <>
struct Mfma<bf16> {
  typedef bf16x8 frag;
  static constexpr int KC = 16;   // K per instruction
  static constexpr int EPL = 8;   // K-values per lane
  __device__ __forceinline__ static f32x16 run(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static frag load(const void* p) { return *reinterpret_cast<const frag*>(p); }
  __device__ __forceinline__ static frag zero() { return frag{}; }
};

template <>
struct Mfma<float> {
  typedef float frag;
  static constexpr int KC = 2;
  static constexpr int EPL = 1;
  __device__ __forceinline__ static f32x16 run(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static frag load(const void* p) { return *reinterpret_cast<const float*>(p); }
  __device__ __forceinline__ static frag zero() { return 0.0f; }
};

// Row of the 32x32 accumulator held in register r by a lane of half `half`.
__device__ __forceinline__ int acc_row(int r, int half) { return 8 * (r >> 2) + 4 * half + (r & 3); }

// Permuted accumulator rows.  If the A operand's row i is loaded from source
// row rperm(i), accumulator register r of lane half h holds source row
// rloc(r, h) = 16 (r / 8) + 8 h + r % 8.  Registers 8c .. 8c+7 of half h then
// cover 8 consecutive source rows 16c + 8h .. 16c + 8h + 7, which is exactly
// the K slot layout of the next MFMA's operand: the accumulator can be fed
// back as an A operand without any data movement.
__device__ __forceinline__ int rloc(int r, int half) { return 16 * (r >> 3) + 8 * half + (r & 7); }
__device__ __forceinline__ int rperm(int i) { return rloc(4 * (i >> 3) + (i & 3), (i >> 2) & 1); }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Operand of a 32x32x16 bf16 MFMA read from a row-major bf16 tile X in LDS
// (`pitch` bytes per row) whose rows are the MFMA's K index: lane l receives
// X[k0 + 8 (l / 32) + e][n0 + l % 32] for e = 0..7.  Uses two gfx950
// transposing reads (ds_read_b64_tr_b16).  Within each 16-lane group, lane
// 4j + p reads 4 consecutive elements of row j and the hardware hands element
// q of lane 4j + p to lane 4p + q as its j-th value.  Addresses are 8-byte
// aligned when n0 is a multiple of 4 and pitch a multiple of 8.
__device__ __forceinline__ bf16x8 lds_tr_frag(const char* tile, int pitch, int k0, int n0, int lane) {
  const int g = lane >> 4, L = lane & 15;
  const int row = k0 + 8 * (g >> 1) + (L >> 2);
  const int colx = n0 + 16 * (g & 1) + 4 * (L & 3);
  const char* a = tile + row * pitch + colx * 2;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a + 4 * pitch));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// A tile of row-major rows held in LDS with no padding: row r occupies
// [r * ROWB, (r + 1) * ROWB) and its 16-byte chunks are permuted by
// chunk' = chunk ^ swz(r), a function of r mod 16.  The permutation makes the
// read patterns of the kernels bank-conflict free on the 64 x 4-byte LDS banks:
//  - 16-byte operand reads, served 16 lanes at a time: 16 rows (in order, or
//    in the rperm order) at one logical chunk, so swz must be one-to-one on
//    16 rows;
//  - transposing 8-byte reads, served 32 lanes at a time: 4 consecutive rows
//    (aligned to 4) x 4 consecutive chunks (aligned to 4), so those 4 rows must
//    move the chunk group (swz >> 2) to 4 different places.
// For 256-byte rows swz swaps the two 2-bit halves of r mod 16; 128-byte rows
// share a bank cycle in pairs, so r's lowest bit is left out.  fp32 tiles
// (512-byte rows, only read one float per lane) stay unpermuted.
template <int ROWB>
struct SwzTile {
  static constexpr int CPR = ROWB / 16;  // 16-byte chunks per row
  __device__ __forceinline__ static int swz(int r) {
    if constexpr (CPR == 16) return ((r & 3) << 2) | ((r >> 2) & 3);
    else if constexpr (CPR == 8) return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
    else return 0;
  }
  // Byte offset of logical byte `colb` of row r.
  __device__ __forceinline__ static int off(int r, int colb) {
    return r * ROWB + ((((colb >> 4) ^ swz(r)) << 4) | (colb & 15));
  }
};

// Direct global -> LDS loads (gfx950 global_load_lds_dwordx4: lane i of a wave
// writes its 16 bytes at the instruction's LDS base + 16 i, no registers) of
// rows [j0, j0 + ROWS) of a row-major global tensor with row stride `rs`
// bytes into a SwzTile<ROWB>.  Rows at or past `nrows` re-read the last row
// (callers mask them out).  The 4 waves of the workgroup split the work; the
// data is in LDS once each wave has waited for its loads (vmcnt 0) and the
// workgroup has passed a barrier.
template <int ROWS, int ROWB>
__device__ __forceinline__ void tile_load_async(char* tile, const char* g, int64_t rs, int j0, int nrows, int wave,
                                                int lane) {
  using TL = SwzTile<ROWB>;
  constexpr int RPI = 1024 / ROWB;      // rows per wave instruction
  constexpr int NI = ROWS / RPI;        // instructions per tile
  static_assert(NI % 4 == 0, "tile must split evenly over 4 waves");
  // Uniform 64-bit row base plus a 32-bit per-lane offset (the host keeps
  // ROWS * rs below 2^31, and row indices below 2^30).
  const char* const base = g + (int64_t)j0 * rs;
  const int rmax = nrows - 1 - j0 < ROWS - 1 ? nrows - 1 - j0 : ROWS - 1;
  const int pc = lane % TL::CPR;
  const int irs = (int)rs;
#pragma unroll
  for (int k = 0; k < NI / 4; ++k) {
    const int m = wave + 4 * k;
    const int r = m * RPI + lane / TL::CPR;
    const int lc = pc ^ TL::swz(r);
    const int rr = r < rmax ? r : rmax;
    const unsigned off = (unsigned)(rr * irs + lc * 16);  // non-negative: scalar-base addressing
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(base + off),
                                     (__attribute__((address_space(3))) void*)(tile + m * 1024), 16, 0, 0);
  }
}

// A pointer that has the same value in every lane of the wave, made visibly
// uniform (held in scalar registers), so that address arithmetic on it stays
// scalar and memory instructions can take it as their scalar base.
__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return reinterpret_cast<const char*>(((uint64_t)hi << 32) | lo);
}

// One direct global -> LDS load of 16 bytes per lane (gfx950
// global_load_lds_dwordx4): lane i writes at lds + 16 i.
__device__ __forceinline__ void global_load_lds16(const char* g, char* lds) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}

// A condition that has the same value in every lane of the wave, made visibly
// uniform: branches on it become scalar branches instead of per-lane
// predication (the compiler cannot tell that values derived from tid >> 6 are
// uniform).
__device__ __forceinline__ bool wave_uniform(bool c) { return __builtin_amdgcn_readfirstlane((int)c) != 0; }

// Wait until this wave's outstanding global loads (including direct-to-LDS
// ones) have landed: s_waitcnt vmcnt(0).
__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// a ^ b evaluated where it is written.  The volatile asm keeps the compiler
// from hoisting per-chunk LDS addresses out of a loop as invariants (each
// would hold a VGPR for the whole loop); b is a constant kept in an SGPR.
__device__ __forceinline__ int xor_here(int a, int b) {
  int r;
  asm volatile("v_xor_b32 %0, %1, %2" : "=v"(r) : "s"(b), "v"(a));
  return r;
}

// Per-lane parts of the LDS addresses of a bf16 SwzTile (ROWB = 128 or 256).
// The chunk XOR and the row base never share bits, so every address is
// (one per-lane base) ^ (a chunk constant) + (a block/stage constant).
template <int ROWB>
struct SwzAddr {
  using TL = SwzTile<ROWB>;
  int afrag;     // A/B-operand fragment of row `r`: offset of chunk 2c + half is afrag ^ (c << 5)
  int tr[2];     // transposing read t: offset for column block cb is tr[t] ^ (cb << 6)
  __device__ __forceinline__ SwzAddr(int r, int half, int lane) {
    afrag = r * ROWB + ((half ^ TL::swz(r)) << 4);
    const int g = lane >> 4, L = lane & 15;
    const int cl = 2 * (g & 1) + ((L & 3) >> 1);  // chunk within a 32-column block
    const int lo = 8 * (L & 1);                   // byte within the chunk
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int row = 8 * (g >> 1) + (L >> 2) + 4 * t;
      tr[t] = row * ROWB + ((cl ^ TL::swz(row)) << 4) + lo;
    }
  }
  // The same addresses in a buffer `bytes` further on (a multiple of 1024, so
  // it commutes with the chunk XOR).  Taking the stage of a double buffer into
  // the per-lane base once per step leaves only constants to be added at each
  // read, which the LDS instructions take as immediate offsets.
  __device__ __forceinline__ SwzAddr shifted(int bytes) const {
    SwzAddr o = *this;
    o.afrag += bytes;
    o.tr[0] += bytes;
    o.tr[1] += bytes;
    return o;
  }
  // 16-byte A/B fragment, K chunk c, of rows starting at block base `blk` (bytes, multiple of 16 rows).
  __device__ __forceinline__ bf16x8 frag(const char* tile, int blk, int c) const {
    return *reinterpret_cast<const bf16x8*>(tile + blk + xor_here(afrag, c << 5));
  }
  // Transposing-read operand (rows k0.. of the tile = blk, columns 32 cb ..).
  __device__ __forceinline__ bf16x8 trfrag(const char* tile, int blk, int cb) const {
    const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + blk + xor_here(tr[0], cb << 6)));
    const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + blk + xor_here(tr[1], cb << 6)));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    const s16x8 v = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
    return __builtin_bit_cast(bf16x8, v);
  }
};

// Transposing-read operand (see lds_tr_frag) from a SwzTile of bf16 rows.
template <int ROWB>
__device__ __forceinline__ bf16x8 lds_tr_frag_swz(const char* tile, int k0, int n0, int lane) {
  using TL = SwzTile<ROWB>;
  const int g = lane >> 4, L = lane & 15;
  const int row = k0 + 8 * (g >> 1) + (L >> 2);
  const int colb = 2 * (n0 + 16 * (g & 1) + 4 * (L & 3));
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + TL::off(row, colb)));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + TL::off(row + 4, colb)));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// 16-byte copy global -> LDS through registers.
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }  // RNE (v_cvt_pk_bf16_f32)
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }

// Clamp a 64-bit index difference into int range for 32-bit mask compares.
__device__ __forceinline__ int clamp_i32(int64_t x) {
  return (int)(x < -(int64_t(1) << 30) ? -(int64_t(1) << 30) : (x > (int64_t(1) << 30) ? (int64_t(1) << 30) : x));
}

// Map a linear workgroup id so that consecutive logical tiles land on the same
// XCD: the hardware hands workgroup i to XCD i % 8, so logical tile
// x * (G / 8) + k is given to workgroup 8 * k + x.  Tiles of one head then run
// together on one XCD and share its L2.
__device__ __forceinline__ int64_t xcd_remap(int64_t bid, int64_t grid) {
  constexpr int kXcds = 8;
  if (grid % kXcds != 0) return bid;
  return (bid % kXcds) * (grid / kXcds) + bid / kXcds;
}

}  // namespace skl
