// Router of the DeepSeekMoE layer (DeepSeekMoE explainer, section "Routing in
// a classic MoE layer"; selection rule of "Top-k routing, from affinities to
// gates"; statistics of "Expert-level balance loss").
//
// One workgroup (4 waves) routes a block of 64 tokens:
//   1. logits u^T e_i: bf16 MFMA 16x16x32 (fp32 accumulate), each wave owns
//      16 tokens and all experts; fp32 storage uses plain FMA dot products;
//   2. a quad of lanes per token does the softmax (max-subtracted) and the
//      top-k selection on the fp32 logits (descending, ties to the lower
//      index), writing indices and gates s_i;
//   3. per-block partial sums of s_i (ascending token) for P;
//   4. a wave ballot per expert gives the block histogram and each
//      (token, slot)'s rank among the block's tokens that picked the same
//      expert, which the scan turns into a stable grouping.
#include "common.h"
#include "kernels.h"

#include <math.h>

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr size_t kDefaultLds = 64 * 1024;  // dynamic LDS allowed without an attribute

struct RouteSmem {
  float* lg;     // [64][ldl] logits; later reused as int ranks
  float* mz;     // [64][2] max and softmax denominator
  int* sidx;     // [64][k] kept experts (-1 for tokens past T)
  int ldl;
};

__device__ __forceinline__ RouteSmem carve(char* smem, int n, int k) {
  RouteSmem s;
  s.ldl = n + 1;
  s.lg = reinterpret_cast<float*>(smem);
  s.mz = s.lg + kRouteTok * s.ldl;
  s.sidx = reinterpret_cast<int*>(s.mz + 2 * kRouteTok);
  return s;
}

size_t route_smem_bytes(int n, int k) {
  return sizeof(float) * (size_t)kRouteTok * (n + 1) + sizeof(float) * 2 * kRouteTok +
         sizeof(int) * (size_t)kRouteTok * k;
}

// Block histogram and in-block ranks.  Every wave sees all 64 tokens (lane =
// token) and handles the experts e = wave, wave + 4, ...
__device__ void block_hist_rank(const RouteSmem& s, int n, int k, int64_t blk, int64_t T,
                                int32_t* blk_cnt, int32_t* lrank) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint64_t bits0 = 0, bits1 = 0, bits2 = 0, bits3 = 0;
  for (int j = 0; j < k; ++j) {
    const int e = s.sidx[lane * k + j];
    if (e < 0) continue;
    const uint64_t b = 1ull << (e & 63);
    switch (e >> 6) {
      case 0: bits0 |= b; break;
      case 1: bits1 |= b; break;
      case 2: bits2 |= b; break;
      default: bits3 |= b; break;
    }
  }
  int* rk = reinterpret_cast<int*>(s.lg);
  const uint64_t below = (1ull << lane) - 1ull;
  for (int e = wave; e < n; e += 4) {
    const int w = e >> 6;
    const uint64_t word = w == 0 ? bits0 : (w == 1 ? bits1 : (w == 2 ? bits2 : bits3));
    const bool has = (word >> (e & 63)) & 1ull;
    const uint64_t mask = __ballot(has);
    if (lane == 0) blk_cnt[blk * n + e] = __popcll(mask);
    if (has) rk[lane * s.ldl + e] = __popcll(mask & below);
  }
  __syncthreads();
  for (int p = tid; p < kRouteTok * k; p += kThreads) {
    const int tl = p / k, j = p - tl * k;
    const int64_t t = blk * kRouteTok + tl;
    const int e = s.sidx[tl * k + j];
    if (t < T) lrank[t * k + j] = e >= 0 ? rk[tl * s.ldl + e] : 0;
  }
}

// bf16 logits with MFMA 16x16x32.  NB = expert blocks of 16 (compile time).
template <int NB>
__device__ void logits_bf16(const uint16_t* __restrict__ u, const uint16_t* __restrict__ cent,
                            int64_t T, int d, int n, int64_t blk, const RouteSmem& s) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, kq = (lane >> 4) * 8;
  int64_t ta = blk * kRouteTok + wave * 16 + r16;
  if (ta > T - 1) ta = T - 1;
  const uint16_t* ap = u + ta * d + kq;
  const uint16_t* cp[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    int e = nb * 16 + r16;
    if (e > n - 1) e = n - 1;
    cp[nb] = cent + (int64_t)e * d + kq;
  }
  f32x4 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
  for (int k0 = 0; k0 < d; k0 += 32) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(ap + k0);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(cp[nb] + k0);
      acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[nb], 0, 0, 0);
    }
  }
  // C layout: lane holds rows 4*(lane/16) + j, column lane % 16.
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int col = nb * 16 + r16;
    if (col < n) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = wave * 16 + (lane >> 4) * 4 + j;
        s.lg[row * s.ldl + col] = acc[nb][j];
      }
    }
  }
}

__device__ void logits_f32(const float* __restrict__ u, const float* __restrict__ cent,
                           int64_t T, int d, int n, int64_t blk, const RouteSmem& s) {
  for (int p = threadIdx.x; p < kRouteTok * n; p += kThreads) {
    const int tl = p / n, e = p - tl * n;
    int64_t t = blk * kRouteTok + tl;
    if (t > T - 1) t = T - 1;
    const float* a = u + t * d;
    const float* b = cent + (int64_t)e * d;
    float acc = 0.f;
    for (int j = 0; j < d; ++j) acc = fmaf(a[j], b[j], acc);
    s.lg[tl * s.ldl + e] = acc;
  }
}

// Softmax, top-k, P partials, histogram.  Logits are already in s.lg.
__device__ void route_tail(int64_t T, int n, int k, int64_t blk, const RouteSmem& s,
                           int32_t* __restrict__ topk_idx, float* __restrict__ topk_gate,
                           int32_t* __restrict__ blk_cnt, float* __restrict__ blk_P,
                           int32_t* __restrict__ lrank) {
  const int tid = threadIdx.x;
  {
    const int tl = tid >> 2, q = tid & 3;
    const int64_t t = blk * kRouteTok + tl;
    const bool valid = t < T;
    const float* row = s.lg + tl * s.ldl;
    float mx = -INFINITY;
    for (int i = q; i < n; i += 4) mx = fmaxf(mx, row[i]);
    mx = fmaxf(mx, __shfl_xor(mx, 1));
    mx = fmaxf(mx, __shfl_xor(mx, 2));
    float z = 0.f;
    for (int i = q; i < n; i += 4) z += expf(row[i] - mx);
    z += __shfl_xor(z, 1);
    z += __shfl_xor(z, 2);
    if (q == 0) {
      s.mz[2 * tl] = mx;
      s.mz[2 * tl + 1] = z;
    }
    // k rounds of a quad arg-max over the experts not taken yet; each lane
    // scans its experts q, q+4, ... in ascending order, so a strict '>'
    // keeps the lower index among equal logits.
    uint64_t taken = 0;
    for (int j = 0; j < k; ++j) {
      float bv = -INFINITY;
      int bi = 0x7fffffff;
      int r = 0;
      for (int i = q; i < n; i += 4, ++r) {
        if ((taken >> r) & 1ull) continue;
        const float v = row[i];
        if (v > bv) {
          bv = v;
          bi = i;
        }
      }
#pragma unroll
      for (int off = 1; off <= 2; off <<= 1) {
        const float ov = __shfl_xor(bv, off);
        const int oi = __shfl_xor(bi, off);
        if (ov > bv || (ov == bv && oi < bi)) {
          bv = ov;
          bi = oi;
        }
      }
      if ((bi & 3) == q) taken |= 1ull << (bi >> 2);
      if (q == 0) {
        s.sidx[tl * k + j] = valid ? bi : -1;
        if (valid) {
          topk_idx[t * k + j] = bi;
          topk_gate[t * k + j] = expf(bv - mx) / z;
        }
      }
    }
  }
  __syncthreads();
  // P partial of this block, tokens ascending.
  for (int i = tid; i < n; i += kThreads) {
    float acc = 0.f;
    for (int tl = 0; tl < kRouteTok; ++tl) {
      if (blk * kRouteTok + tl >= T) break;
      acc += expf(s.lg[tl * s.ldl + i] - s.mz[2 * tl]) / s.mz[2 * tl + 1];
    }
    blk_P[blk * n + i] = acc;
  }
  __syncthreads();
  block_hist_rank(s, n, k, blk, T, blk_cnt, lrank);
}

template <int NB>
__global__ __launch_bounds__(kThreads) void route_bf16_kernel(
    const uint16_t* __restrict__ u, const uint16_t* __restrict__ cent, int64_t T, int d, int n,
    int k, int32_t* __restrict__ topk_idx, float* __restrict__ topk_gate,
    int32_t* __restrict__ blk_cnt, float* __restrict__ blk_P, int32_t* __restrict__ lrank) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const RouteSmem s = carve(smem, n, k);
  const int64_t blk = blockIdx.x;
  logits_bf16<NB>(u, cent, T, d, n, blk, s);
  __syncthreads();
  route_tail(T, n, k, blk, s, topk_idx, topk_gate, blk_cnt, blk_P, lrank);
}

__global__ __launch_bounds__(kThreads) void route_f32_kernel(
    const float* __restrict__ u, const float* __restrict__ cent, int64_t T, int d, int n, int k,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_gate,
    int32_t* __restrict__ blk_cnt, float* __restrict__ blk_P, int32_t* __restrict__ lrank) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const RouteSmem s = carve(smem, n, k);
  const int64_t blk = blockIdx.x;
  logits_f32(u, cent, T, d, n, blk, s);
  __syncthreads();
  route_tail(T, n, k, blk, s, topk_idx, topk_gate, blk_cnt, blk_P, lrank);
}

__global__ __launch_bounds__(kThreads) void hist_kernel(const int32_t* __restrict__ topk_idx,
                                                        int64_t T, int n, int k,
                                                        int32_t* __restrict__ blk_cnt,
                                                        int32_t* __restrict__ lrank) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const RouteSmem s = carve(smem, n, k);
  const int64_t blk = blockIdx.x;
  for (int p = threadIdx.x; p < kRouteTok * k; p += kThreads) {
    const int tl = p / k, j = p - tl * k;
    const int64_t t = blk * kRouteTok + tl;
    const int e = t < T ? topk_idx[t * k + j] : -1;
    s.sidx[p] = (e >= 0 && e < n) ? e : -1;
  }
  __syncthreads();
  block_hist_rank(s, n, k, blk, T, blk_cnt, lrank);
}

// ---------------------------------------------------------------- scans

// Exclusive scan of v[0..cnt) in LDS by the first `cnt` threads' values;
// returns the exclusive prefix for this thread and stores the total.
// All threads of the block must call it.  buf holds >= 1024 ints.
__device__ int block_exclusive_scan(int v, int cnt, int* buf, int* total) {
  const int tid = threadIdx.x;
  const int nt = blockDim.x;
  buf[tid] = tid < cnt ? v : 0;
  __syncthreads();
  for (int off = 1; off < nt; off <<= 1) {
    const int add = tid >= off ? buf[tid - off] : 0;
    __syncthreads();
    buf[tid] += add;
    __syncthreads();
  }
  const int incl = buf[tid];
  if (tid == nt - 1) *total = incl;
  __syncthreads();
  return incl - (tid < cnt ? v : 0);
}

// Writes the M-tiles of group g (rows cnt starting at grouped row first).
__device__ __forceinline__ void emit_tiles(const TileList& tl, int first_tile, int first_row,
                                           int cnt) {
  int tile = first_tile;
  for (int r = 0; r < cnt && tile < tl.max_tiles; r += kTileM, ++tile) {
    tl.row0[tile] = first_row + r;
    tl.rows[tile] = cnt - r < kTileM ? cnt - r : kTileM;
  }
}

constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(kScanThreads) void scan_kernel(
    const int32_t* __restrict__ blk_cnt, const float* __restrict__ blk_P, int B, int64_t T,
    int n, int k, int32_t* __restrict__ counts, float* __restrict__ f, float* __restrict__ P,
    int32_t* __restrict__ offsets, int32_t* __restrict__ blk_base, TileList tl, int has_tiles) {
  __shared__ int csum[kScanThreads];
  __shared__ float psum[kScanThreads];
  __shared__ int sbuf[kScanThreads];
  __shared__ int s_cnt[kMaxExperts];
  __shared__ int s_off[kMaxExperts];
  __shared__ int s_total;
  const int tid = threadIdx.x;
  int C = kScanThreads / n;
  if (C > B) C = B;
  if (C < 1) C = 1;
  const int per = (B + C - 1) / C;
  const int e = tid % n, c = tid / n;
  const bool act = c < C;
  const int b0 = c * per, b1 = (c + 1) * per < B ? (c + 1) * per : B;
  if (act) {
    int cs = 0;
    float ps = 0.f;
    for (int b = b0; b < b1; ++b) {
      cs += blk_cnt[(int64_t)b * n + e];
      if (blk_P) ps += blk_P[(int64_t)b * n + e];
    }
    csum[c * n + e] = cs;
    psum[c * n + e] = ps;
  }
  __syncthreads();
  if (tid < n) {
    int run = 0;
    float pr = 0.f;
    for (int cc = 0; cc < C; ++cc) {
      const int v = csum[cc * n + tid];
      csum[cc * n + tid] = run;
      run += v;
      pr += psum[cc * n + tid];
    }
    s_cnt[tid] = run;
    if (counts) counts[tid] = run;
    if (f) f[tid] = (float)((int64_t)run * n) / (float)((int64_t)k * T);
    if (P && blk_P) P[tid] = pr / (float)T;
  }
  __syncthreads();
  const int cnt_e = tid < n ? s_cnt[tid] : 0;
  const int off_e = block_exclusive_scan(cnt_e, n, sbuf, &s_total);
  if (tid < n) {
    s_off[tid] = off_e;
    offsets[tid] = off_e;
  }
  if (tid == 0) offsets[n] = s_total;
  __syncthreads();
  if (has_tiles) {
    const int nt_e = tid < n ? (cnt_e + kTileM - 1) / kTileM : 0;
    const int toff = block_exclusive_scan(nt_e, n, sbuf, &s_total);
    if (tid < n) {
      tl.off[tid] = toff;
      emit_tiles(tl, toff, off_e, cnt_e);
    }
    if (tid == 0) {
      tl.off[n] = s_total;
      *tl.count = s_total;
    }
  }
  if (act) {
    int base = s_off[e] + csum[c * n + e];
    for (int b = b0; b < b1; ++b) {
      blk_base[(int64_t)b * n + e] = base;
      base += blk_cnt[(int64_t)b * n + e];
    }
  }
}

constexpr int kTileThreads = 256;

// Offsets that break the documented contract (decreasing, outside
// [0, rows]) are clamped so that every tile stays inside the row range and
// the tile capacity.
__global__ __launch_bounds__(kTileThreads) void tiles_kernel(const int32_t* __restrict__ offsets,
                                                             int G, int64_t rows, TileList tl) {
  __shared__ int sbuf[kTileThreads];
  __shared__ int s_total;
  const int tid = threadIdx.x;
  int first = 0, cnt = 0;
  if (tid < G) {
    const int64_t a = offsets[tid], b = offsets[tid + 1];
    const int64_t lo = a < 0 ? 0 : (a > rows ? rows : a);
    const int64_t hi = b < lo ? lo : (b > rows ? rows : b);
    first = (int)lo;
    cnt = (int)(hi - lo);
  }
  const int nt_g = (cnt + kTileM - 1) / kTileM;
  const int toff = block_exclusive_scan(nt_g, G, sbuf, &s_total);
  if (tid < G) {
    tl.off[tid] = toff;
    emit_tiles(tl, toff, first, cnt);
  }
  if (tid == 0) {
    const int total = s_total < tl.max_tiles ? s_total : tl.max_tiles;
    tl.off[G] = total;
    *tl.count = total;
  }
}

}  // namespace

hipError_t launch_route(int dtype, const void* u, const void* cent, int64_t T, int d, int n,
                        int k, int32_t* topk_idx, float* topk_gate, int32_t* blk_cnt,
                        float* blk_P, int32_t* lrank, hipStream_t s) {
  const int B = (int)((T + kRouteTok - 1) / kRouteTok);
  const size_t sm = route_smem_bytes(n, k);
  if (dtype == 0) {
    if (sm > kDefaultLds) {
      const hipError_t e = hipFuncSetAttribute((const void*)route_f32_kernel,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(route_f32_kernel, dim3(B), dim3(kThreads), sm, s, (const float*)u,
                       (const float*)cent, T, d, n, k, topk_idx, topk_gate, blk_cnt, blk_P,
                       lrank);
    return hipGetLastError();
  }
  const int nb = (n + 15) / 16;
#define MOE_ROUTE_CASE(NBV)                                                                    \
  {                                                                                            \
    if (sm > kDefaultLds) {                                                                    \
      const hipError_t e = hipFuncSetAttribute((const void*)route_bf16_kernel<NBV>,            \
                                               hipFuncAttributeMaxDynamicSharedMemorySize,     \
                                               (int)sm);                                       \
      if (e != hipSuccess) return e;                                                           \
    }                                                                                          \
    hipLaunchKernelGGL(route_bf16_kernel<NBV>, dim3(B), dim3(kThreads), sm, s,                 \
                       (const uint16_t*)u, (const uint16_t*)cent, T, d, n, k, topk_idx,        \
                       topk_gate, blk_cnt, blk_P, lrank);                                      \
  }
  if (nb <= 1) MOE_ROUTE_CASE(1)
  else if (nb <= 2) MOE_ROUTE_CASE(2)
  else if (nb <= 4) MOE_ROUTE_CASE(4)
  else if (nb <= 8) MOE_ROUTE_CASE(8)
  else MOE_ROUTE_CASE(16)
#undef MOE_ROUTE_CASE
  return hipGetLastError();
}

hipError_t launch_hist(const int32_t* topk_idx, int64_t T, int n, int k, int32_t* blk_cnt,
                       int32_t* lrank, hipStream_t s) {
  const int B = (int)((T + kRouteTok - 1) / kRouteTok);
  const size_t sm = route_smem_bytes(n, k);
  if (sm > kDefaultLds) {
    const hipError_t e = hipFuncSetAttribute((const void*)hist_kernel,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(hist_kernel, dim3(B), dim3(kThreads), sm, s, topk_idx,
                     T, n, k, blk_cnt, lrank);
  return hipGetLastError();
}

hipError_t launch_scan(const int32_t* blk_cnt, const float* blk_P, int64_t T, int n, int k,
                       int32_t* counts, float* f, float* P, int32_t* offsets, int32_t* blk_base,
                       const TileList* tiles, hipStream_t s) {
  const int B = (int)((T + kRouteTok - 1) / kRouteTok);
  TileList tl = tiles ? *tiles : TileList{nullptr, nullptr, nullptr, nullptr, 0};
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kScanThreads), 0, s, blk_cnt, blk_P, B, T, n, k,
                     counts, f, P, offsets, blk_base, tl, tiles ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_tiles(const int32_t* offsets, int n_groups, int64_t rows,
                        const TileList& tiles, hipStream_t s) {
  hipLaunchKernelGGL(tiles_kernel, dim3(1), dim3(kTileThreads), 0, s, offsets, n_groups, rows,
                     tiles);
  return hipGetLastError();
}

}  // namespace moe
