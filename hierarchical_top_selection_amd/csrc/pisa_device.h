// pisa_device.h - device-side building blocks shared by the gfx950 kernels.
//
// MFMA operand layout (verified on gfx950 for v_mfma_f32_16x16x32_bf16 and
// v_mfma_f32_16x16x4_f32): lane l of the wave supplies row (l % 16) of the
// 16-row A tile and column (l % 16) of the 16-column B tile, covering the
// k-slice owned by its lane group g = l / 16; the 16x16 fp32 result gives
// lane l column (l % 16) and rows 4 * g + i, i = 0..3.  Because A and B use
// the same k-slice per lane, any bijection between (k-step, g) and the
// contraction index is valid as long as both operands use it; the loaders
// below pick the bijection that makes each lane's loads contiguous.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pisa {

constexpr int kLeaf = 64;      // C: keys per leaf block
constexpr int kFanout = 2;     // g: children per node above the leaves
constexpr int kMaxLevels = 32;
constexpr float kNegInf = -__builtin_huge_valf();

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// ----------------------------------------------------------------------------- geometry
// Level sizes for the current length and node offsets for the capacity layout.
struct Levels {
  int count;                   // levels for the current length: L(n)
  int size[kMaxLevels];        // size[l-1] = M_l(n)
  int64_t offset[kMaxLevels];  // node offset of level l in the capacity layout
  int64_t nodes;               // nodes per (b, kvh) in the capacity layout
};

__host__ __device__ inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

// First key covered by node i of level l (level 1 = leaves).
__device__ inline int64_t node_first_key(int level, int64_t i) {
  return i * (int64_t)kLeaf << (level - 1);
}

// ----------------------------------------------------------------------------- element I/O
__device__ inline float to_f32(float x) { return x; }
__device__ inline float to_f32(__bf16 x) { return (float)x; }

template <typename T> __device__ inline T from_f32(float x);
template <> __device__ inline float from_f32<float>(float x) { return x; }
template <> __device__ inline __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }  // RNE

// Four consecutive elements starting at p (p 8-byte aligned for bf16, 16-byte for f32).
__device__ inline float4 load4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ inline float4 load4(const __bf16* p) {
  bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
  return make_float4((float)v[0], (float)v[1], (float)v[2], (float)v[3]);
}

// ----------------------------------------------------------------------------- MFMA fragments
// Row fragment of a 16 x D operand tile for the fp32 MFMA (16x16x4): the lane
// holds, for m = 0..D/16-1, the four contraction indices 16 m + 4 g + j, which
// feed k-steps 4 m + j.
template <int D>
struct FragF32 {
  static constexpr int kVecs = D / 16;       // 16-byte pieces per lane
  // element offset (within a row) of piece m for lane group g
  __host__ __device__ static constexpr int piece_offset(int m, int g) { return 16 * m + 4 * g; }
  float4 v[D / 16];
  template <typename T>
  __device__ inline void load(const T* row, int g) {
#pragma unroll
    for (int m = 0; m < D / 16; ++m) v[m] = load4(row + 16 * m + 4 * g);
  }
  __device__ inline void zero() {
#pragma unroll
    for (int m = 0; m < D / 16; ++m) v[m] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
};

// Row fragment for the bf16 MFMA (16x16x32): k-step s covers indices 32 s + 8 g + j.
template <int D>
struct FragBF16 {
  static constexpr int kVecs = D / 32;       // 16-byte pieces per lane
  // element offset (within a row) of piece s for lane group g
  __host__ __device__ static constexpr int piece_offset(int s, int g) { return 32 * s + 8 * g; }
  bf16x8 v[D / 32];
  __device__ inline void load(const __bf16* row, int g) {
#pragma unroll
    for (int s = 0; s < D / 32; ++s) v[s] = *reinterpret_cast<const bf16x8*>(row + 32 * s + 8 * g);
  }
  __device__ inline void zero() {
#pragma unroll
    for (int s = 0; s < D / 32; ++s)
#pragma unroll
      for (int j = 0; j < 8; ++j) v[s][j] = (__bf16)0.f;
  }
};

// Row fragment for the f16 MFMA (16x16x32): same element placement as FragBF16.
template <int D>
struct FragF16 {
  f16x8 v[D / 32];
  __device__ inline void load(const _Float16* row, int g) {
#pragma unroll
    for (int s = 0; s < D / 32; ++s) v[s] = *reinterpret_cast<const f16x8*>(row + 32 * s + 8 * g);
  }
};

__device__ inline floatx4 mfma_f32(float a, float b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ inline floatx4 mfma_bf16(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// acc += A(16 x D) * B(D x 16) with both operands as row fragments.
template <int D>
__device__ inline floatx4 mma(const FragF32<D>& a, const FragF32<D>& b, floatx4 acc) {
#pragma unroll
  for (int m = 0; m < D / 16; ++m) {
    acc = mfma_f32(a.v[m].x, b.v[m].x, acc);
    acc = mfma_f32(a.v[m].y, b.v[m].y, acc);
    acc = mfma_f32(a.v[m].z, b.v[m].z, acc);
    acc = mfma_f32(a.v[m].w, b.v[m].w, acc);
  }
  return acc;
}
template <int D>
__device__ inline floatx4 mma(const FragBF16<D>& a, const FragBF16<D>& b, floatx4 acc) {
#pragma unroll
  for (int s = 0; s < D / 32; ++s) acc = mfma_bf16(a.v[s], b.v[s], acc);
  return acc;
}
template <int D>
__device__ inline floatx4 mma(const FragF16<D>& a, const FragF16<D>& b, floatx4 acc) {
#pragma unroll
  for (int s = 0; s < D / 32; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a.v[s], b.v[s], acc, 0, 0, 0);
  return acc;
}

// Fragment type used for raw Q/K contractions of element type T.
template <typename T, int D> struct RawFrag;
template <int D> struct RawFrag<float, D> { typedef FragF32<D> type; };
template <int D> struct RawFrag<__bf16, D> { typedef FragBF16<D> type; };

// Index of the calling wave within its workgroup, as a wave-uniform (scalar) value: the
// compiler cannot tell that threadIdx.x / 64 is uniform, and everything derived from it
// (token, item and loop bounds) would otherwise live in vector registers and take
// exec-masked branches.
__device__ inline int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// ----------------------------------------------------------------------------- wave reductions
__device__ inline float wave_max_xor(float x, int mask) { return fmaxf(x, __shfl_xor(x, mask, 64)); }
__device__ inline float wave_add_xor(float x, int mask) { return x + __shfl_xor(x, mask, 64); }

// Max / sum over the four 16-lane rows (lanes l, l ^ 16, l ^ 32, l ^ 48), every lane getting the
// result, with the gfx950 row-swap permutes instead of LDS shuffles.  With both operands equal to
// x, v_permlane16_swap leaves rows (r0, r0, r2, r2) in the first and (r1, r1, r3, r3) in the
// second register, v_permlane32_swap the low half twice and the high half twice.  Sums come out
// as (r0 + r1) + (r2 + r3) in every lane, the order of the xor-shuffle pair above.  The permutes
// are written in asm because the compiler folds the two results of its builtins into one when
// the operands are the same value; a permute reads its registers two wait states after the VALU
// write, hence the s_nop on each side.
__device__ inline void swap_rows16(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ inline void swap_rows32(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ inline float rows_max(float x) {
  float a = x, b = x;
  swap_rows16(a, b);
  a = fmaxf(a, b);
  b = a;
  swap_rows32(a, b);
  return fmaxf(a, b);
}
__device__ inline float rows_sum(float x) {
  float a = x, b = x;
  swap_rows16(a, b);
  a = a + b;
  b = a;
  swap_rows32(a, b);
  return a + b;
}

// Sum over the 16 lanes of each row (lanes 16 r .. 16 r + 15) with DPP row shifts;
// the row total lands in the row's last lane (lane 16 r + 15).
__device__ inline float row_sum_to_last(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x111, 0xf, 0xf, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x112, 0xf, 0xf, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x114, 0xf, 0xf, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x118, 0xf, 0xf, true));
  return x;
}

// Orders this wave's LDS writes before its later LDS reads of other lanes' data
// (wave-private staging buffers; no workgroup barrier needed).
__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// ----------------------------------------------------------------------------- candidate scores
// Score of a candidate from the raw dot products y0, y1 of its two children (valid where ok0 /
// ok1), "Block Sparse Attention with Log-Linear Complexity", Core method: mode 0 is the LSE of
// eq. 21, returned in base-2 units (logits y * c2, c2 = scale * log2 e); modes 1 and 2 are its
// first- and second-order Taylor truncations (PISA-1 / PISA-2): the mean, and the mean plus half
// the population variance, of the logits y * scale, in natural units.  -inf without a valid child.
__device__ inline float pair_score(float y0, float y1, bool ok0, bool ok1, int mode, float scale, float c2) {
  if (mode == 0) {
    const float z0 = ok0 ? y0 * c2 : kNegInf, z1 = ok1 ? y1 * c2 : kNegInf;
    const float m = fmaxf(z0, z1);
    return m == kNegInf ? kNegInf : m + __builtin_amdgcn_logf(1.f + __builtin_amdgcn_exp2f(fminf(z0, z1) - m));
  }
  if (!(ok0 || ok1)) return kNegInf;
  const float a = y0 * scale, b = y1 * scale;
  if (!(ok0 && ok1)) return ok0 ? a : b;
  const float mean = 0.5f * (a + b), h = 0.5f * (a - b);
  return mode == 2 ? mean + 0.5f * h * h : mean;
}

// Keep flag of lane i's candidate among the wave's K best by (score descending, index ascending).
// khi is the candidate's score bits made order-preserving (0 for an empty lane, above 0 for every
// valid one), and the valid lanes hold ascending indices, so among equal scores the lower lane is
// the lower index.  Needs more than K valid lanes.  A bitwise search from the top bit finds the
// K-th largest khi as the largest threshold that at least K lanes reach; every lane above it is
// kept, and the lowest lanes equal to it fill the places that remain.
__device__ inline bool keep_top_k(uint32_t khi, int k) {
  uint32_t thr = 0;
#pragma unroll
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t trial = thr | (1u << bit);
    if (__popcll(__ballot(khi >= trial)) >= k) thr = trial;
  }
  const uint64_t ties = __ballot(khi == thr);
  const int need = k - __popcll(__ballot(khi > thr));
  const int before = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(ties >> 32),
                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)ties, 0u));
  return khi > thr || (khi == thr && before < need);
}

// Order-preserving bits of a score (-0 as +0) for keep_top_k; 0 for an empty lane.
__device__ inline uint32_t score_key(float u, bool valid) {
  const uint32_t ub = __builtin_bit_cast(uint32_t, u + 0.f);
  return valid ? ((ub & 0x80000000u) ? ~ub : (ub | 0x80000000u)) : 0u;
}

// Index of the p-th set bit (p counted from 0) of a non-empty 64-bit mask.
__device__ inline int nth_set_bit(uint64_t mask, int p) {
  int pos = 0;
#pragma unroll
  for (int step = 32; step > 0; step >>= 1) {
    const int k = pos + step;
    const uint64_t below = k >= 64 ? mask : (mask & ((1ull << k) - 1ull));
    if (__popcll(below) <= p) pos = k;
  }
  return pos;
}

}  // namespace pisa
