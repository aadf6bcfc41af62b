// Grouping of (token, slot) pairs by expert and the gate-weighted combine.
//
// Grouping follows the page's note that a production layer groups tokens per
// expert (DeepSeekMoE explainer, "Top-k routing, from affinities to gates"):
// row position = expert offset + rows of earlier token blocks for the expert
// (scan) + rank inside the token block (wave ballot), i.e. a stable counting
// sort.  The combine forms h = sum_j g_j FFN_j(u) + shared + u of section
// "Routing in a classic MoE layer".
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kScatterThreads = 256;  // one wave per token

__global__ __launch_bounds__(kScatterThreads) void scatter_kernel(
    const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ lrank,
    const int32_t* __restrict__ blk_base, int64_t T, int n, int k,
    int32_t* __restrict__ perm_token, int32_t* __restrict__ slot_of,
    const uint8_t* __restrict__ u, uint8_t* __restrict__ x_perm, int row_bytes) {
  __shared__ int spos[4][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + wave;
  if (t >= T) return;  // whole wave leaves together
  const int64_t R = T * k;
  if (lane < k) {
    // Expert ids outside [0, n) break the documented contract; such slots
    // are left out (slot_of = -1) rather than indexing out of range.
    const int e = topk_idx[t * k + lane];
    int pos = -1;
    if (e >= 0 && e < n) {
      pos = blk_base[(t / kRouteTok) * blk_ld(n) + e] + lrank[t * k + lane];
      if (pos < 0 || pos >= R) pos = -1;
    }
    slot_of[t * k + lane] = pos;
    if (pos >= 0) perm_token[pos] = (int32_t)t;
    spos[wave][lane] = pos;
  }
  if (!x_perm) return;
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  const int nch = row_bytes / 16;
  const u32x4* src = reinterpret_cast<const u32x4*>(u + t * row_bytes);
  for (int c = lane; c < nch; c += 64) {
    const u32x4 v = src[c];
    for (int j = 0; j < k; ++j) {
      const int64_t pj = spos[wave][j];
      if (pj >= 0) reinterpret_cast<u32x4*>(x_perm + pj * row_bytes)[c] = v;
    }
  }
}

constexpr int kCombineThreads = 256;

// Eight consecutive elements of a row, loaded whole (16 bytes of bf16, 32 of
// fp32) and read back as fp32.
template <typename T>
struct Chunk;
template <>
struct Chunk<uint16_t> {
  u32x4 v;
  static __device__ __forceinline__ Chunk load(const uint16_t* p) {
    return Chunk{*reinterpret_cast<const u32x4*>(p)};
  }
  __device__ __forceinline__ float get(int i) const {
    const uint32_t w = v[i >> 1];
    return bf16_to_f32((uint16_t)((i & 1) ? (w >> 16) : (w & 0xFFFFu)));
  }
};
template <>
struct Chunk<float> {
  u32x4 a, b;
  static __device__ __forceinline__ Chunk load(const float* p) {
    return Chunk{*reinterpret_cast<const u32x4*>(p), *reinterpret_cast<const u32x4*>(p + 4)};
  }
  __device__ __forceinline__ float get(int i) const {
    return __uint_as_float(i < 4 ? a[i] : b[i - 4]);
  }
};

// One workgroup per token; each thread owns chunks of 8 elements.
template <int DT>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(
    const typename Elem<DT>::T* __restrict__ residual,
    const typename Elem<DT>::T* __restrict__ shared_out,
    const typename Elem<DT>::T* __restrict__ y, const int32_t* __restrict__ slot_of,
    const float* __restrict__ gate, typename Elem<DT>::T* __restrict__ h, int d, int k) {
  typedef Elem<DT> E;
  __shared__ int s_slot[64];
  __shared__ float s_g[64];
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  if (tid < k) {
    // slot ids come from the grouping; clamp so a malformed one cannot index
    // outside y_perm
    const int64_t R = (int64_t)gridDim.x * k;
    int64_t v = slot_of[t * k + tid];
    v = v < 0 ? 0 : (v >= R ? R - 1 : v);
    s_slot[tid] = (int)v;
    s_g[tid] = gate[t * k + tid];
  }
  __syncthreads();
  const int nch = d / 8;
  for (int c = tid; c < nch; c += kCombineThreads) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    // The chunk's shared and residual rows and up to kBatch gathered rows
    // are loaded before any is summed, so a token costs one memory round
    // trip per kBatch slots (the sum keeps the order: slots ascending, then
    // shared, then residual).
    typedef typename E::T ET;
    constexpr int kBatch = 8;
    Chunk<ET> sh{}, rs{};
    if (shared_out) sh = Chunk<ET>::load(shared_out + t * d + c * 8);
    if (residual) rs = Chunk<ET>::load(residual + t * d + c * 8);
    for (int j0 = 0; j0 < k; j0 += kBatch) {
      Chunk<ET> v[kBatch];
#pragma unroll
      for (int jj = 0; jj < kBatch; ++jj)
        if (j0 + jj < k) v[jj] = Chunk<ET>::load(y + (int64_t)s_slot[j0 + jj] * d + c * 8);
#pragma unroll
      for (int jj = 0; jj < kBatch; ++jj) {
        if (j0 + jj < k) {
          const float g = s_g[j0 + jj];
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] += g * v[jj].get(i);
        }
      }
    }
    if (shared_out) {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += sh.get(i);
    }
    if (residual) {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += rs.get(i);
    }
    typename E::T* out = h + t * d + c * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) E::st(out, i, acc[i]);
  }
}

}  // namespace

hipError_t launch_scatter(const int32_t* topk_idx, const int32_t* lrank,
                          const int32_t* blk_base, int64_t T, int n, int k,
                          int32_t* perm_token, int32_t* slot_of, const void* u, void* x_perm,
                          int row_bytes, hipStream_t s) {
  const int64_t grid = (T + 3) / 4;
  hipLaunchKernelGGL(scatter_kernel, dim3((unsigned)grid), dim3(kScatterThreads), 0, s, topk_idx,
                     lrank, blk_base, T, n, k, perm_token, slot_of, (const uint8_t*)u,
                     (uint8_t*)x_perm, row_bytes);
  return hipGetLastError();
}

hipError_t launch_combine(int dtype, const void* residual, const void* shared_out,
                          const void* y_perm, const int32_t* slot_of, const float* gate,
                          void* h, int64_t T, int d, int k, hipStream_t s) {
  if (dtype == 0) {
    hipLaunchKernelGGL(combine_kernel<0>, dim3((unsigned)T), dim3(kCombineThreads), 0, s,
                       (const float*)residual, (const float*)shared_out, (const float*)y_perm,
                       slot_of, gate, (float*)h, d, k);
  } else {
    hipLaunchKernelGGL(combine_kernel<1>, dim3((unsigned)T), dim3(kCombineThreads), 0, s,
                       (const uint16_t*)residual, (const uint16_t*)shared_out,
                       (const uint16_t*)y_perm, slot_of, gate, (uint16_t*)h, d, k);
  }
  return hipGetLastError();
}

}  // namespace moe
