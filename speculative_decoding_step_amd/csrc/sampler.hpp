// Integer-weight sampling helpers shared by the draft's chain draws and the
// acceptance samplers.  A distribution w over the vocabulary is drawn from
// with W_v = floor(w_v * 2^48) and r = floor(u * sum W): the pick is the first
// v whose inclusive prefix sum exceeds r, so it does not depend on summation
// order.  Rows are cut into slices of SAMPLE_SLICE entries: a grid-wide pass
// writes each slice's sum, and the pick reads the slice sums, finds the slice
// holding r and scans that slice only.
#pragma once

#include <hip/hip_runtime.h>

namespace e3 {

constexpr int SAMPLE_SLICE = 4096;  // vocabulary entries per slice
inline int sampler_slices(int V) { return (V + SAMPLE_SLICE - 1) / SAMPLE_SLICE; }

// floor(p(v) * 2^48), p(v) = fl32(exp(z_v / T - lse)) (lse in double)
__device__ __forceinline__ float sample_prob(const float* z, int v, double temp, double lse) {
  return (float)exp((double)z[v] / temp - lse);
}
__device__ __forceinline__ unsigned long long int_weight_of(float w) { return (unsigned long long)ldexpf(w, 48); }
__device__ __forceinline__ unsigned long long int_weight(const float* z, int v, double temp, double lse) {
  return int_weight_of(sample_prob(z, v, temp, lse));
}

// floor(u * S) for u = uu / 2^24, exact in 64 bits
__device__ __forceinline__ unsigned long long floor_u_times(unsigned long long S, unsigned long long uu) {
  return (S >> 24) * uu + (((S & 0xffffffull) * uu) >> 24);
}
__device__ __forceinline__ unsigned long long uniform24(float u) { return (unsigned long long)(u * 16777216.0f); }

// Block-wide inclusive prefix sum of one value per thread (blockDim.x == 1024):
// sc[tid] receives the prefix, the total is returned to every thread.
__device__ inline unsigned long long block_prefix(unsigned long long* sc, unsigned long long x) {
  const int tid = threadIdx.x;
  __syncthreads();  // earlier readers of sc are done
  sc[tid] = x;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const unsigned long long add = tid >= o ? sc[tid - o] : 0ull;
    __syncthreads();
    sc[tid] += add;
    __syncthreads();
  }
  return sc[1023];
}

// Block-wide (256 threads) sum; every thread receives it.
__device__ inline unsigned long long block_sum256(unsigned long long* red, unsigned long long x) {
  const int tid = threadIdx.x;
  __syncthreads();  // earlier readers of red are done
  red[tid] = x;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) red[tid] += red[tid + o];
    __syncthreads();
  }
  return red[0];
}

}  // namespace e3
