// Device helpers shared by the EAGLE-3 step kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define E3_DEV __device__ __forceinline__

typedef uint16_t bf16_t;  // bfloat16 bits
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- bf16 <-> f32
E3_DEV float bf2f(bf16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// Round to nearest, ties to even (NaN kept quiet).
E3_DEV bf16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

// Storage element access for T = float or bf16_t.
template <typename T> E3_DEV float ld(const T* p, size_t i);
template <> E3_DEV float ld<float>(const float* p, size_t i) { return p[i]; }
template <> E3_DEV float ld<bf16_t>(const bf16_t* p, size_t i) { return bf2f(p[i]); }
template <typename T> E3_DEV void st(T* p, size_t i, float v);
template <> E3_DEV void st<float>(float* p, size_t i, float v) { p[i] = v; }
template <> E3_DEV void st<bf16_t>(bf16_t* p, size_t i, float v) { p[i] = f2bf(v); }

// Four consecutive elements as float4 (16-byte or 8-byte loads/stores).
template <typename T> E3_DEV float4 ld4(const T* p, size_t i);
template <> E3_DEV float4 ld4<float>(const float* p, size_t i) { return *(const float4*)(p + i); }
template <> E3_DEV float4 ld4<bf16_t>(const bf16_t* p, size_t i) {
  const uint2 u = *(const uint2*)(p + i);
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                     __uint_as_float(u.y & 0xffff0000u));
}
template <typename T> E3_DEV void st4(T* p, size_t i, float4 v);
template <> E3_DEV void st4<float>(float* p, size_t i, float4 v) { *(float4*)(p + i) = v; }
template <> E3_DEV void st4<bf16_t>(bf16_t* p, size_t i, float4 v) {
  uint2 u;
  u.x = (uint32_t)f2bf(v.x) | ((uint32_t)f2bf(v.y) << 16);
  u.y = (uint32_t)f2bf(v.z) | ((uint32_t)f2bf(v.w) << 16);
  *(uint2*)(p + i) = u;
}

// ------------------------------------------------ column-slab activations
// Index of element (row r, column k) of an [R, K] matrix stored as column
// slabs of 32: slab k / 32 holds every row's 32 columns of it, row after row
// (64 bytes per row in bf16).  The large-M GEMM reads its activations this
// way: 16 consecutive rows of one slab, one MFMA operand fragment, are one
// contiguous KiB; a kernel that produces one row at a time still writes
// 64-byte pieces.  The inputs of passes of more than 64 rows use it.
E3_DEV size_t slab32_index(int r, int k, int R) { return ((size_t)(k >> 5) * R + r) * 32 + (k & 31); }

// ---------------------------------------------------------------- reductions
E3_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
E3_DEV double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
E3_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Block-wide sum for blockDim.x a multiple of 64 (<= 1024); `red` holds >= 16 floats.
E3_DEV float block_sum(float v, float* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < nw; ++i) t += red[i];
  return t;
}

// Split-K partials: sum over k < S of p[k * stride], added in split order.
// The loads are issued eight at a time so that they are in flight together.
E3_DEV float sum_splits(const float* __restrict__ p, int S, size_t stride) {
  float s = 0.f;
  for (int k0 = 0; k0 < S; k0 += 8) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = (k0 + j < S) ? p[(size_t)(k0 + j) * stride] : 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (k0 + j < S) s += v[j];
  }
  return s;
}

E3_DEV float4 sum_splits4(const float4* __restrict__ p, int S, size_t stride4) {
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int k0 = 0; k0 < S; k0 += 8) {
    float4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = (k0 + j < S) ? p[(size_t)(k0 + j) * stride4] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (k0 + j < S) {
        s.x += v[j].x; s.y += v[j].y; s.z += v[j].z; s.w += v[j].w;
      }
  }
  return s;
}

// (value, index) order used by every top-k and argmax: larger value first,
// lower index on ties.
// Written with non-short-circuit operators so that it compiles to compares and
// mask arithmetic rather than branches.
E3_DEV bool better(float va, int ia, float vb, int ib) {
  return (va > vb) | ((va == vb) & ((unsigned)ia < (unsigned)ib));
}

struct VI {
  float v;
  int i;
};

E3_DEV VI vi_best(VI a, VI b) { return better(a.v, a.i, b.v, b.i) ? a : b; }

// Best (value, index) of a full wave, returned to every lane.  Within each
// 16-lane row: DPP exchanges with lanes xor 1, xor 2 (quad permutes), then the
// half-row and row mirrors; across rows: the gfx950 permlane swaps, which
// hand each lane the value of lane xor 16, then of lane xor 32, in registers
// (no trip through LDS).  The order is a total order, so the result does not
// depend on the reduction tree.  Every lane must be active.
template <int CTRL>
E3_DEV VI vi_dpp(VI a) {
  const VI b{__int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a.v), CTRL, 0xF, 0xF, false)),
             __builtin_amdgcn_update_dpp(0, a.i, CTRL, 0xF, 0xF, false)};
  return vi_best(a, b);
}

// Best (value, index) of each 16-lane row, returned to every lane of the row.
E3_DEV VI row16_best(VI x) {
  x = vi_dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x = vi_dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x = vi_dpp<0x141>(x);  // row_half_mirror
  return vi_dpp<0x140>(x);  // row_mirror
}

// Sum over each 16-lane row (double), returned to every lane of the row.
template <int CTRL>
E3_DEV double dpp_d(double a) {
  const unsigned long long u = __double_as_longlong(a);
  const unsigned lo = __builtin_amdgcn_update_dpp(0u, (unsigned)u, CTRL, 0xF, 0xF, false);
  const unsigned hi = __builtin_amdgcn_update_dpp(0u, (unsigned)(u >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}
E3_DEV double row16_sum_d(double x) {
  x += dpp_d<0xB1>(x);
  x += dpp_d<0x4E>(x);
  x += dpp_d<0x141>(x);
  return x + dpp_d<0x140>(x);
}

// The better of the two (value, index) pairs a permlane swap hands a lane: its own and its partner's.
E3_DEV VI vi_swap16(VI x) {
  const auto v = __builtin_amdgcn_permlane16_swap(__float_as_uint(x.v), __float_as_uint(x.v), false, false);
  const auto i = __builtin_amdgcn_permlane16_swap((unsigned)x.i, (unsigned)x.i, false, false);
  return vi_best(VI{__uint_as_float(v[0]), (int)i[0]}, VI{__uint_as_float(v[1]), (int)i[1]});
}
E3_DEV VI vi_swap32(VI x) {
  const auto v = __builtin_amdgcn_permlane32_swap(__float_as_uint(x.v), __float_as_uint(x.v), false, false);
  const auto i = __builtin_amdgcn_permlane32_swap((unsigned)x.i, (unsigned)x.i, false, false);
  return vi_best(VI{__uint_as_float(v[0]), (int)i[0]}, VI{__uint_as_float(v[1]), (int)i[1]});
}

E3_DEV VI wave_best(VI x) { return vi_swap32(vi_swap16(row16_best(x))); }

// Wave-wide maximum and float64 sum in registers only (DPP within rows, permlane swaps across them); every lane
// must be active.  The sum's lane 0 is the same on every run (a fixed order of additions).
E3_DEV float wave_max_reg(float x) {
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false)));
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
E3_DEV double swap_sum_d(double x, bool wide) {
  const unsigned long long u = __double_as_longlong(x);
  const unsigned lo = (unsigned)u, hi = (unsigned)(u >> 32);
  const auto l = wide ? __builtin_amdgcn_permlane32_swap(lo, lo, false, false)
                      : __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
  const auto h = wide ? __builtin_amdgcn_permlane32_swap(hi, hi, false, false)
                      : __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
  const double a = __longlong_as_double((long long)(((unsigned long long)h[0] << 32) | l[0]));
  const double b = __longlong_as_double((long long)(((unsigned long long)h[1] << 32) | l[1]));
  return a + b;
}
E3_DEV double wave_sum_d_reg(double x) { return swap_sum_d(swap_sum_d(row16_sum_d(x), false), true); }

// Status bits (mirrors eagle3.h).
#define E3_DEV_KV_OVERFLOW 0x1
#define E3_DEV_BAD_TREE 0x2
#define E3_DEV_BAD_TOKEN 0x4
#define E3_DEV_BAD_PATH 0x8

E3_DEV void raise_flag(int* status, int bit) { atomicOr(status, bit); }
