// Device-side building blocks for the libgdn kernels (gfx950 / CDNA4).
//
// MFMA shapes used (lane l of a 64-wide wave, g = l / 16, i = l % 16):
//   bf16  v_mfma_f32_16x16x32_bf16: A[m][k] with m = i, k = 8g..8g+7;
//                                   B[k][n] with k = 8g..8g+7, n = i;
//   fp32  v_mfma_f32_16x16x4_f32:   A[m][k] with m = i, k = g;
//                                   B[k][n] with k = g, n = i;
//   both: C[m][n] with m = 4g + r (r = 0..3 in the four accumulator
//         registers), n = i.
// These lane layouts were checked on gfx950 against a host matmul.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

enum IoKind { IO_BF16 = 0, IO_F32 = 1 };

template <int IO> struct Io;
template <> struct Io<IO_BF16> {
  typedef uint16_t elem;               // raw bf16 bits
  static constexpr int bytes = 2;
  static constexpr int kblock = 32;    // contraction depth of one MFMA
};
template <> struct Io<IO_F32> {
  typedef float elem;
  static constexpr int bytes = 4;
  static constexpr int kblock = 4;
};

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
// The wave index is the same for all lanes of a wave; readfirstlane makes
// that visible to the compiler so per-wave choices compile to scalar
// branches instead of exec-masked ones.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
// fp32 -> bf16 bits, round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }
__device__ __forceinline__ bf16x8 zero_bf16x8() {
  return __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
}

// Eight consecutive bf16 of a row (16 bytes).
__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

// Eight consecutive fp32 values rounded to a bf16 fragment.
__device__ __forceinline__ bf16x8 f32x8_to_bf16x8(const float* v) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = static_cast<__bf16>(v[e]);
  return r;
}

// Column fragment of a row-major bf16 matrix M in LDS (row stride ld
// elements): lane (g, i) receives M[k0 + 8g + e][c0 + i], e = 0..7.
// Uses the gfx950 transposing LDS read: within each group of 16 lanes,
// lane i receives element i % 4 of the 8-byte chunk addressed by lane
// 4j + i / 4 as its element j.  Lane m therefore addresses row
// k0 + 8g + m / 4 (+4 for the second read), columns c0 + 4 (m % 4) .. +3.
// Needs (ld * 2) and (c0 * 2) to be multiples of 8 bytes.
__device__ __forceinline__ bf16x8 lds_col_frag_bf16(const uint16_t* M, int ld, int k0, int c0) {
  const int l = lane_id();
  const int g = l >> 4, m = l & 15;
  const uint16_t* p0 = M + (k0 + 8 * g + (m >> 2)) * ld + c0 + 4 * (m & 3);
  const uint16_t* p1 = p0 + 4 * ld;
  i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
  i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p1));
  i16x8 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, ab);
}

// Four rows of a column of a row-major bf16 matrix M in LDS (row stride ld
// elements), with the gfx950 transposing read: lane (g, i) receives
// M[r0 + j][c0 + i], j = 0..3, where r0 may differ between the four groups
// of 16 lanes.  Lane m of a group addresses row r0 + m / 4, columns
// c0 + 4 (m % 4) .. + 3.  Needs (ld * 2) and (c0 * 2) to be multiples of 8
// bytes.
__device__ __forceinline__ i16x4 lds_rows4_tr(const uint16_t* M, int ld, int r0, int c0) {
  const int m = lane_id() & 15;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(M + (r0 + (m >> 2)) * ld + c0 + 4 * (m & 3)));
}

// Sum over the 16 lanes of v's DPP row (lanes 16r .. 16r + 15), returned to
// all 16 with the same rounding: lane ^ 1, lane ^ 2 (quad permutes), then
// the mirror within each half row and within the row.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp_mov<0xB1>(v);    // quad_perm [1, 0, 3, 2]
  v += dpp_mov<0x4E>(v);    // quad_perm [2, 3, 0, 1]
  v += dpp_mov<0x141>(v);   // row_half_mirror
  v += dpp_mov<0x140>(v);   // row_mirror
  return v;
}
// Sum of squares of the 8 bf16 (or 4 fp32) values of a 16-byte piece, and
// the piece scaled by r (bf16 rounded to nearest even).
template <int IO>
__device__ __forceinline__ float piece_sumsq(const u32x4& v) {
  float ss = 0.f;
  if constexpr (IO == IO_BF16) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float lo = __uint_as_float(v[e] << 16), hi = __uint_as_float(v[e] & 0xffff0000u);
      ss = fmaf(hi, hi, fmaf(lo, lo, ss));
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) ss = fmaf(__uint_as_float(v[e]), __uint_as_float(v[e]), ss);
  }
  return ss;
}
template <int IO>
__device__ __forceinline__ u32x4 piece_scale(const u32x4& v, float r) {
  u32x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if constexpr (IO == IO_BF16) {
      const float lo = __uint_as_float(v[e] << 16) * r;
      const float hi = __uint_as_float(v[e] & 0xffff0000u) * r;
      o[e] = (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
    } else {
      o[e] = __float_as_uint(__uint_as_float(v[e]) * r);
    }
  }
  return o;
}

// Reciprocal of the L2 norm from a sum of squares; 0 for a zero row.
__device__ __forceinline__ float inv_norm(float ss) { return ss > 0.f ? rsqrtf(ss) : 0.f; }

// Block-wide barrier.
__device__ __forceinline__ void block_sync() { __syncthreads(); }

// ---- Direct global -> LDS copies (gfx950 global_load_lds) --------------
// One instruction copies `size` bytes per lane; lane l's bytes land at
// lds_base + size * l (lds_base must be the same for the whole wave).  The
// copies count in the wave's vector-memory counter and complete in issue
// order with its other vector-memory operations; the compiler does not
// track them, so consumers wait explicitly with wait_vm_barrier.
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

__device__ __forceinline__ void dma16(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds((glb_void_t*)(src), (lds_void_t*)(lds_base), 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds((glb_void_t*)(src), (lds_void_t*)(lds_base), 4, 0, 0);
}

// Wait until at most N of this wave's vector-memory operations are still
// outstanding, then barrier the workgroup.  With N no larger than the
// number of copies the wave issued after a given stage, that stage has
// landed for every wave once the barrier is passed.  The empty asm keeps
// the compiler from moving LDS accesses across.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Workgroup barrier for LDS hand-offs only: waits for this wave's LDS
// operations, then barriers.  Unlike __syncthreads it carries no memory
// fence, so it does not wait for global loads still in flight (a
// prefetch ring stays in flight across it).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((63 & 15) | ((63 >> 4) << 14) | (7 << 4) | (0 << 8));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// XCD-aware work ordering.  Hardware hands consecutive workgroup ids to the
// 8 XCDs in turn; this maps them so that each XCD receives a contiguous
// range of work items (neighbouring heads of the same frame share L2 there).
__device__ __forceinline__ int xcd_item(int id, int total) {
  const int per = total >> 3, rem = total & 7;
  const int x = id & 7, local = id >> 3;
  return x * per + (x < rem ? x : rem) + local;
}

}  // namespace gdn
