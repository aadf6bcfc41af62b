// Router of the DeepSeekMoE layer (DeepSeekMoE explainer, section "Routing in
// a classic MoE layer"; selection rule of "Top-k routing, from affinities to
// gates"; statistics of "Expert-level balance loss").
//
// One workgroup (8 waves) routes a block of 16 tokens:
//   1. logits u^T e_i: bf16 MFMA 16x16x32 (fp32 accumulate); the 8 waves
//      split the hidden dimension so each issues its loads in one batch,
//      and their partial logits are added in a fixed order; fp32 storage
//      uses plain FMA dot products;
//   2. one 16-lane DPP row per token does the softmax (max-subtracted) and
//      the top-k selection on the fp32 logits (descending, ties to the lower
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

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kTailThreads = kRouteTok * 16;  // 16 lanes (one DPP row) per token
constexpr size_t kDefaultLds = 64 * 1024;    // dynamic LDS allowed without an attribute

struct RouteSmem {
  float* part;   // [4][16][ldl] partial logits (waves w and w+4 share slot w)
  float* lg;     // [16][ldl] logits; later reused as int ranks
  float* sv;     // [16][ldl] softmax values
  int* sidx;     // [16][k] kept experts (-1 for tokens past T)
  int ldl;
};

__device__ __forceinline__ RouteSmem carve(char* smem, int n) {
  RouteSmem s;
  s.ldl = n + 1;
  s.part = reinterpret_cast<float*>(smem);
  s.lg = s.part + 4 * kRouteTok * s.ldl;
  s.sv = s.lg + kRouteTok * s.ldl;
  s.sidx = reinterpret_cast<int*>(s.sv + kRouteTok * s.ldl);
  return s;
}

size_t route_smem_bytes(int n, int k) {
  return sizeof(float) * (size_t)6 * kRouteTok * (n + 1) + sizeof(int) * (size_t)kRouteTok * k;
}
__host__ __device__ inline size_t route_smem_bytes_aligned(int n, int k) {
  return ((sizeof(float) * (size_t)6 * kRouteTok * (n + 1) + sizeof(int) * (size_t)kRouteTok * k) +
          15) & ~(size_t)15;
}

// Cross-lane moves inside a 16-lane DPP row (VALU latency, no LDS crossbar).
template <int CTRL>
__device__ __forceinline__ int dpp(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
  return __int_as_float(dpp<CTRL>(__float_as_int(v)));
}
// Butterfly over a row: xor 1, xor 2 (quad permutes), then the half-row and
// row mirrors pair the quads and the half-rows; every lane ends with the
// reduction of all 16.
constexpr int kQuadX1 = 0xB1, kQuadX2 = 0x4E, kHalfMirror = 0x141, kMirror = 0x140;

__device__ __forceinline__ float row_max(float v) {
  v = fmaxf(v, dppf<kQuadX1>(v));
  v = fmaxf(v, dppf<kQuadX2>(v));
  v = fmaxf(v, dppf<kHalfMirror>(v));
  return fmaxf(v, dppf<kMirror>(v));
}
__device__ __forceinline__ float row_sum(float v) {
  v += dppf<kQuadX1>(v);
  v += dppf<kQuadX2>(v);
  v += dppf<kHalfMirror>(v);
  return v + dppf<kMirror>(v);
}
// Selection keys: the logit's bits made order-preserving as an unsigned
// integer (-0 folded into +0 first, so equal values give equal high words)
// above the complement of the expert index.  Larger key = larger logit, and
// among equal logits the lower index; 0 is below every real key and marks a
// taken or absent expert.  Keys are unique, so an unsigned max is the rule's
// arg-max with no tie branch.
__device__ __forceinline__ uint64_t topk_key(float v, int i) {
  uint32_t b = __float_as_uint(v + 0.0f);
  b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((uint64_t)b << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)i);
}
__device__ __forceinline__ int topk_key_index(uint64_t key) {
  return (int)(0xFFFFFFFFu - (uint32_t)key);
}
__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }
template <int CTRL>
__device__ __forceinline__ uint64_t dpp64(uint64_t x) {
  const uint32_t lo = (uint32_t)dpp<CTRL>((int)(uint32_t)x);
  const uint32_t hi = (uint32_t)dpp<CTRL>((int)(uint32_t)(x >> 32));
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t row_max_key(uint64_t x) {
  x = umax64(x, dpp64<kQuadX1>(x));
  x = umax64(x, dpp64<kQuadX2>(x));
  x = umax64(x, dpp64<kHalfMirror>(x));
  return umax64(x, dpp64<kMirror>(x));
}

// Block histogram and in-block ranks.  Lanes 0..15 of waves 0..HW-1 stand
// for the block's 16 tokens; wave w handles the experts e = w, w + HW, ...
// (the route kernel's upper waves sum P meanwhile: HW = 4 there).
template <int HW = kWaves>
__device__ void block_hist_rank(const RouteSmem& s, int n, int k, int64_t blk, int64_t T,
                                int32_t* blk_cnt, int32_t* lrank) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint64_t bits0 = 0, bits1 = 0, bits2 = 0, bits3 = 0;
  if (wave < HW && lane < kRouteTok) {
    for (int j = 0; j < k; ++j) {
      const int e = s.sidx[lane * k + j];
      const uint64_t b = e >= 0 ? 1ull << (e & 63) : 0ull;
      const int w = e >> 6;
      bits0 |= w == 0 ? b : 0ull;
      bits1 |= w == 1 ? b : 0ull;
      bits2 |= w == 2 ? b : 0ull;
      bits3 |= w >= 3 ? b : 0ull;
    }
  }
  int* rk = reinterpret_cast<int*>(s.lg);
  const uint64_t below = (1ull << lane) - 1ull;
  const int ldn = blk_ld(n);
  for (int e = wave; wave < HW && e < n; e += HW) {
    const int w = e >> 6;
    const uint64_t word = w == 0 ? bits0 : (w == 1 ? bits1 : (w == 2 ? bits2 : bits3));
    const bool has = (word >> (e & 63)) & 1ull;
    const uint64_t mask = __ballot(has);
    if (lane == 0) blk_cnt[blk * ldn + e] = __popcll(mask);
    if (has) rk[lane * s.ldl + e] = __popcll(mask & below);
  }
  if (tid < ldn - n) blk_cnt[blk * ldn + n + tid] = 0;
  __syncthreads();
  for (int p = tid; p < kRouteTok * k; p += kThreads) {
    const int tl = p / k, j = p - tl * k;
    const int64_t t = blk * kRouteTok + tl;
    const int e = s.sidx[tl * k + j];
    if (t < T) lrank[t * k + j] = e >= 0 ? rk[tl * s.ldl + e] : 0;
  }
}

// bf16 logits with MFMA 16x16x32.  NB = expert blocks of 16 (compile time).
// Wave w accumulates the 32-wide hidden slices [w*S/8, (w+1)*S/8), loading a
// chunk of U slices before its MFMAs.
// Partial logits of the 8 waves (each over its hidden slices) into s.lg.
// C layout: lane holds rows 4*(lane/16) + j, column lane % 16.  Waves 4..7
// store first, waves 0..3 add theirs on top, then the four slots are added
// in a fixed order.
template <int NB>
__device__ __forceinline__ void reduce_partials(const f32x4 (&acc)[NB], int n, const RouteSmem& s) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15;
  const int stride = kRouteTok * s.ldl;
  float* part = s.part + (wave & 3) * stride;
  if (wave >= 4) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int col = nb * 16 + r16;
      if (col < n) {
#pragma unroll
        for (int j = 0; j < 4; ++j) part[((lane >> 4) * 4 + j) * s.ldl + col] = acc[nb][j];
      }
    }
  }
  __syncthreads();
  if (wave < 4) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int col = nb * 16 + r16;
      if (col < n) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float* q = part + ((lane >> 4) * 4 + j) * s.ldl + col;
          *q = acc[nb][j] + *q;
        }
      }
    }
  }
  __syncthreads();
  for (int p = tid; p < kRouteTok * n; p += kThreads) {
    const int tl = p / n, e = p - tl * n;
    const int o = tl * s.ldl + e;
    s.lg[o] = ((s.part[o] + s.part[stride + o]) + s.part[2 * stride + o]) + s.part[3 * stride + o];
  }
}

template <int NB>
__device__ void logits_bf16(const uint16_t* __restrict__ u, const uint16_t* __restrict__ cent,
                            int64_t T, int d, int n, int64_t blk, const RouteSmem& s) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, kq = (lane >> 4) * 8;
  int64_t ta = blk * kRouteTok + r16;
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
  const int S = d / 32;
  const int s0 = wave * S / kWaves, s1 = (wave + 1) * S / kWaves;
  constexpr int U = NB <= 4 ? 8 : (NB <= 8 ? 4 : 2);
  int st = s0;
  for (; st + U <= s1; st += U) {
    bf16x8 a[U], b[U][NB];
#pragma unroll
    for (int uu = 0; uu < U; ++uu) {
      a[uu] = *reinterpret_cast<const bf16x8*>(ap + (st + uu) * 32);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        b[uu][nb] = *reinterpret_cast<const bf16x8*>(cp[nb] + (st + uu) * 32);
    }
    // Keep the whole batch in flight: without this fence the scheduler trades
    // it for a short sliding window to save registers.
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int uu = 0; uu < U; ++uu)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[uu], b[uu][nb], acc[nb], 0, 0, 0);
  }
  for (; st < s1; ++st) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(ap + st * 32);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(cp[nb] + st * 32);
      acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[nb], 0, 0, 0);
    }
  }
  reduce_partials<NB>(acc, n, s);
}

// bf16 logits with the hidden dimension staged through LDS (n <= 64, and
// d <= 2048 so a wave's slices fit one round of loads).  Each wave reads
// its hidden range in chunks of two 32-wide slices; one load instruction
// covers 8 rows x 128 contiguous bytes (whole cache lines, where the MFMA
// operand layout would read 16 rows x 64 bytes), every chunk of the wave is
// in flight at once, and the wave rewrites each chunk into MFMA operand
// order in its own LDS region: [activations: 2 blocks][centroids: NB x 2
// blocks] of 64 lanes x 16 bytes.  Same MFMAs, same per-wave slice order
// and the same reduction as logits_bf16, so the logits are identical.
constexpr int kStageChunks = 4;  // chunks of two slices per wave (d <= 2048)

// 16-byte slot j of an operand block lives at slot j ^ (((j >> 4) & 7) << 1):
// a permutation inside every 64-slot block that spreads both the staging
// writes (8 rows x 8 pieces per instruction) and the operand reads (64
// consecutive slots) over all bank groups.
__device__ __forceinline__ uint32_t stage_slot(uint32_t j) { return j ^ (((j >> 4) & 7u) << 1); }

template <int NB>
__device__ __forceinline__ int stage_region_bytes() {
  return (2 + 2 * NB) * 1024;
}

template <int NB>
__device__ void logits_bf16_staged(const uint16_t* __restrict__ u,
                                   const uint16_t* __restrict__ cent, int64_t T, int d, int n,
                                   int64_t blk, const RouteSmem& s, char* stage) {
  constexpr int kLdB = 2 * NB;    // centroid load instructions per chunk
  constexpr int kLd = kLdB + 2;   // + 2 for the 16 token rows
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  char* reg = stage + wave * stage_region_bytes<NB>();
  const int S = d / 32;
  const int s0 = wave * S / kWaves, s1 = (wave + 1) * S / kWaves;
  const int nsl = s1 - s0;         // this wave's slices (at most 8)
  const int nch = (nsl + 1) >> 1;  // chunks of two slices
  const int lr8 = lane >> 3, pc = lane & 7;
  uint32_t go[kLd], wo[kLd];       // global byte offsets (chunk 0), LDS byte offsets
#pragma unroll
  for (int i = 0; i < kLd; ++i) {
    const int r = (i < kLdB ? i : i - kLdB) * 8 + lr8;  // centroid row / token row
    const int L = (r & 15) + 16 * (pc & 3), uu = pc >> 2;
    if (i < kLdB) {
      const int e = r < n ? r : n - 1;
      go[i] = ((uint32_t)e * (uint32_t)d + (uint32_t)(s0 * 32 + pc * 8)) * 2u;
      wo[i] = 2048u + stage_slot((uint32_t)(((r >> 4) * 2 + uu) * 64 + L)) * 16u;
    } else {
      int64_t t = blk * kRouteTok + r;
      if (t > T - 1) t = T - 1;
      go[i] = ((uint32_t)t * (uint32_t)d + (uint32_t)(s0 * 32 + pc * 8)) * 2u;
      wo[i] = stage_slot((uint32_t)(uu * 64 + L)) * 16u;
    }
  }
  u32x4 buf[kStageChunks][kLd];
#pragma unroll
  for (int c = 0; c < kStageChunks; ++c) {
    // pieces past the wave's last slice (odd slice count) are not read
    const bool ok = c < nch && 64 * c + pc * 8 < nsl * 32;
#pragma unroll
    for (int i = 0; i < kLd; ++i)
      buf[c][i] = ok ? ld_off<u32x4>(i < kLdB ? cent : u, go[i] + (uint32_t)c * 128u)
                     : u32x4{0u, 0u, 0u, 0u};
  }
  f32x4 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < kStageChunks; ++c) {
    if (c < nch) {
#pragma unroll
      for (int i = 0; i < kLd; ++i) *reinterpret_cast<u32x4*>(reg + wo[i]) = buf[c][i];
      // the wave reads what its other lanes wrote
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int uu = 0; uu < 2; ++uu) {
        if (2 * c + uu < nsl) {
          const bf16x8 a =
              *reinterpret_cast<const bf16x8*>(reg + stage_slot((uint32_t)(uu * 64 + lane)) * 16);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            const bf16x8 b = *reinterpret_cast<const bf16x8*>(
                reg + 2048 + stage_slot((uint32_t)((nb * 2 + uu) * 64 + lane)) * 16);
            acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[nb], 0, 0, 0);
          }
        }
      }
      // reads done before the next chunk overwrites the region
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
  reduce_partials<NB>(acc, n, s);
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

// Softmax and top-k of one token on a 16-lane DPP row.  Lane q of the row
// keeps the logits of experts q, q+16, ... (NB of them) in registers, so the
// k selection rounds touch no memory.  Writes the softmax values to srow and
// the kept experts to sidx (-1 when the token is past T) and, for a real
// token t, its topk_idx / topk_gate row.
template <int NB>
__device__ __forceinline__ void token_topk(const float* row, float* srow, int* sidx, int q, int n,
                                           int k, bool valid, int64_t t,
                                           int32_t* __restrict__ topk_idx,
                                           float* __restrict__ topk_gate) {
  float v[NB];
#pragma unroll
  for (int r = 0; r < NB; ++r) {
    const int i = q + 16 * r;
    v[r] = i < n ? row[i] : -INFINITY;
  }
  float mx = v[0];
#pragma unroll
  for (int r = 1; r < NB; ++r) mx = fmaxf(mx, v[r]);
  mx = row_max(mx);
  float ev[NB];
  float z = 0.f;
#pragma unroll
  for (int r = 0; r < NB; ++r) {
    ev[r] = q + 16 * r < n ? expf(v[r] - mx) : 0.f;
    z += ev[r];
  }
  z = row_sum(z);
  // one correctly rounded reciprocal, then a product per expert (one more
  // rounding than a division, far inside the gates' bar)
  const float rz = 1.0f / z;
#pragma unroll
  for (int r = 0; r < NB; ++r)
    if (q + 16 * r < n) srow[q + 16 * r] = ev[r] * rz;
  // k rounds of a row arg-max over the selection keys (larger logit, then
  // lower index); the winner's key becomes 0 in the lane that holds it.
  uint64_t key[NB];
#pragma unroll
  for (int r = 0; r < NB; ++r) key[r] = q + 16 * r < n ? topk_key(v[r], q + 16 * r) : 0ull;
  for (int j = 0; j < k; ++j) {
    uint64_t best = key[0];
#pragma unroll
    for (int r = 1; r < NB; ++r) best = umax64(best, key[r]);
    best = row_max_key(best);
#pragma unroll
    for (int r = 0; r < NB; ++r) key[r] = key[r] == best ? 0ull : key[r];
    if (q == 0) sidx[j] = valid ? topk_key_index(best) : -1;
  }
  // The row's lanes write the kept experts and their gates together (the
  // rounds above carry no memory wait).
  if (valid)
    for (int j = q; j < k; j += 16) {
      const int e = sidx[j];
      topk_idx[t * k + j] = e;
      topk_gate[t * k + j] = srow[e];
    }
}

// Softmax, top-k, P partials, histogram.  Logits are already in s.lg.
template <int NB>
__device__ void route_tail(int64_t T, int n, int k, int64_t blk, const RouteSmem& s,
                           int32_t* __restrict__ topk_idx, float* __restrict__ topk_gate,
                           int32_t* __restrict__ blk_cnt, float* __restrict__ blk_P,
                           int32_t* __restrict__ lrank) {
  const int tid = threadIdx.x;
  if (tid < kTailThreads) {  // whole waves
    const int tl = tid >> 4;
    const int64_t t = blk * kRouteTok + tl;
    token_topk<NB>(s.lg + tl * s.ldl, s.sv + tl * s.ldl, s.sidx + tl * k, tid & 15, n, k, t < T,
                   t, topk_idx, topk_gate);
  }
  __syncthreads();
  // P partial of this block, tokens ascending (waves 4..7, while waves 0..3
  // form the histogram).
  const int ldn = blk_ld(n);
  for (int i = tid - kThreads / 2; i >= 0 && i < ldn; i += kThreads / 2) {
    float acc = 0.f;
    if (i < n) {
      float vals[kRouteTok];
#pragma unroll
      for (int tl = 0; tl < kRouteTok; ++tl)
        vals[tl] = blk * kRouteTok + tl < T ? s.sv[tl * s.ldl + i] : 0.f;
#pragma unroll
      for (int tl = 0; tl < kRouteTok; ++tl) acc += vals[tl];
    }
    blk_P[blk * ldn + i] = acc;
  }
  block_hist_rank<kWaves / 2>(s, n, k, blk, T, blk_cnt, lrank);
}

template <int NB, bool STAGED>
__global__ __launch_bounds__(kThreads) void route_bf16_kernel(
    const uint16_t* __restrict__ u, const uint16_t* __restrict__ cent, int64_t T, int d, int n,
    int k, int32_t* __restrict__ topk_idx, float* __restrict__ topk_gate,
    int32_t* __restrict__ blk_cnt, float* __restrict__ blk_P, int32_t* __restrict__ lrank,
    float* __restrict__ lg_out, int ld_out) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const RouteSmem s = carve(smem, n);
  const int64_t blk = blockIdx.x;
  if constexpr (STAGED)
    logits_bf16_staged<NB>(u, cent, T, d, n, blk, s, smem + route_smem_bytes_aligned(n, k));
  else
    logits_bf16<NB>(u, cent, T, d, n, blk, s);
  __syncthreads();
  if (lg_out) {  // the logits for a backward pass, rows padded with zeros to ld_out
    for (int i = threadIdx.x; i < kRouteTok * ld_out; i += kThreads) {
      const int tl = i / ld_out, e = i - tl * ld_out;
      const int64_t t = blk * kRouteTok + tl;
      if (t < T) lg_out[t * ld_out + e] = e < n ? s.lg[tl * s.ldl + e] : 0.0f;
    }
  }
  route_tail<NB>(T, n, k, blk, s, topk_idx, topk_gate, blk_cnt, blk_P, lrank);
}

template <int NB>
__global__ __launch_bounds__(kThreads) void route_f32_kernel(
    const float* __restrict__ u, const float* __restrict__ cent, int64_t T, int d, int n, int k,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_gate,
    int32_t* __restrict__ blk_cnt, float* __restrict__ blk_P, int32_t* __restrict__ lrank) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const RouteSmem s = carve(smem, n);
  const int64_t blk = blockIdx.x;
  logits_f32(u, cent, T, d, n, blk, s);
  __syncthreads();
  route_tail<NB>(T, n, k, blk, s, topk_idx, topk_gate, blk_cnt, blk_P, lrank);
}

__global__ __launch_bounds__(kThreads) void hist_kernel(const int32_t* __restrict__ topk_idx,
                                                        int64_t T, int n, int k,
                                                        int32_t* __restrict__ blk_cnt,
                                                        int32_t* __restrict__ lrank) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const RouteSmem s = carve(smem, n);
  const int64_t blk = blockIdx.x;
  for (int p = threadIdx.x; p < kRouteTok * k; p += kThreads) {
    const int tl = p / k, j = p - tl * k;
    const int64_t t = blk * kRouteTok + tl;
    const int e = t < T ? topk_idx[t * k + j] : -1;
    s.sidx[p] = (e >= 0 && e < n) ? e : -1;
  }
  __syncthreads();
  block_hist_rank<kWaves>(s, n, k, blk, T, blk_cnt, lrank);
}

// ---------------------------------------------------------------- scans

// Exclusive scan over the first 256 threads (4 whole waves) of one value
// each; every thread of the block must call it.  wsum holds >= 4 ints.
__device__ int scan256(int v, int* wsum, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int incl = v;
  if (tid < 256) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    if (lane == 63) wsum[wave] = incl;
  }
  __syncthreads();
  int pre = 0;
  if (tid < 256)
    for (int w = 0; w < wave; ++w) pre += wsum[w];
  if (tid == 255) *total = pre + incl;
  __syncthreads();
  return pre + incl - v;
}

// M-tile list from expert totals (s_cnt) and offsets (s_off, n + 1 entries)
// held in LDS; s_toff is n + 1 ints of LDS scratch.  Every thread of the
// block must call it.
__device__ void emit_tile_list(const TileList& tl, int n, const int* s_cnt, const int* s_off,
                               int* s_toff, int* wsum, int* s_total, int nthreads) {
  const int tid = threadIdx.x;
  const int cnt_e = tid < n ? s_cnt[tid] : 0;
  const int toff = scan256((cnt_e + kTileM - 1) / kTileM, wsum, s_total);
  if (tid < n) {
    s_toff[tid] = toff;
    tl.off[tid] = toff;
  }
  if (tid == 0) {
    s_toff[n] = *s_total;
    tl.off[n] = *s_total;
    *tl.count = *s_total;
  }
  if (tl.steal && tid < 16) tl.steal[tid] = 0;
  __syncthreads();
  // Tile t belongs to the last expert whose first tile is <= t.
  const int total = s_toff[n];
  for (int t = tid; t < total && t < tl.max_tiles; t += nthreads) {
    int lo = 0, hi = n;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_toff[mid] <= t)
        lo = mid;
      else
        hi = mid;
    }
    const int r = (t - s_toff[lo]) * kTileM;
    tl.row0[t] = s_off[lo] + r;
    tl.rows[t] = s_cnt[lo] - r < kTileM ? s_cnt[lo] - r : kTileM;
  }
}

// Writes the M-tiles of one group (rows cnt starting at grouped row first).
__device__ __forceinline__ void emit_tiles(const TileList& tl, int first_tile, int first_row,
                                           int cnt) {
  int tile = first_tile;
  for (int r = 0; r < cnt && tile < tl.max_tiles; r += kTileM, ++tile) {
    tl.row0[tile] = first_row + r;
    tl.rows[tile] = cnt - r < kTileM ? cnt - r : kTileM;
  }
}

constexpr int kScanThreads = 1024;
constexpr int kScanRows = 8;  // 16-byte rows a thread keeps in registers

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i32x4 shfl_up4(i32x4 v, int off, int width) {
  return i32x4{__shfl_up(v.x, off, width), __shfl_up(v.y, off, width), __shfl_up(v.z, off, width),
               __shfl_up(v.w, off, width)};
}
__device__ __forceinline__ f32x4v shfl_xor4(f32x4v v, int m, int width) {
  return f32x4v{__shfl_xor(v.x, m, width), __shfl_xor(v.y, m, width), __shfl_xor(v.z, m, width),
                __shfl_xor(v.w, m, width)};
}

// Column scan of the [B][ldn] block histograms.  Thread (e4, c) owns the
// four experts 4*e4 .. 4*e4+3 (one 16-byte column) over a chunk of
// consecutive blocks; the C chunks of a column are C consecutive lanes
// (C a power of two dividing 64), so the prefix over chunks and the column
// totals are lane shuffles.  Counts stay in registers between the sum and
// the write of the per-block bases.  Integer sums are exact in any order;
// the P sums run rows ascending inside a chunk, then a fixed butterfly.
__global__ __launch_bounds__(kScanThreads) void scan_kernel(
    const int32_t* __restrict__ blk_cnt, const float* __restrict__ blk_P, int B, int64_t T,
    int n, int k, int32_t* __restrict__ counts, float* __restrict__ f, float* __restrict__ P,
    int32_t* __restrict__ offsets, int32_t* __restrict__ blk_base, TileList tl, int has_tiles) {
  __shared__ int s_cnt[kMaxExperts];
  __shared__ float s_P[kMaxExperts];
  __shared__ int s_off[kMaxExperts + 1];
  __shared__ int s_toff[kMaxExperts + 1];
  __shared__ int wsum[4];
  __shared__ int s_total;
  const int tid = threadIdx.x;
  const int ldn = blk_ld(n), n4 = ldn >> 2;
  int cmax = kScanThreads / n4;
  if (cmax > 64) cmax = 64;
  if (cmax > B) cmax = B;
  int C = 1;
  while (C * 2 <= cmax) C *= 2;
  const int per = (B + C - 1) / C;
  const int e4 = tid / C, c = tid - (tid / C) * C;
  const bool act = e4 < n4;
  const int b0 = c * per < B ? c * per : B;
  const int b1 = b0 + per < B ? b0 + per : B;
  const bool cached = per <= kScanRows;
  const int64_t col = 4 * e4;
  i32x4 v[kScanRows];
  i32x4 cs = {0, 0, 0, 0};
  f32x4v ps = {0.f, 0.f, 0.f, 0.f};
  if (act) {
    if (cached) {
#pragma unroll
      for (int i = 0; i < kScanRows; ++i) {
        v[i] = b0 + i < b1 ? *reinterpret_cast<const i32x4*>(blk_cnt + (int64_t)(b0 + i) * ldn + col)
                           : i32x4{0, 0, 0, 0};
        cs += v[i];
      }
      if (blk_P) {
        f32x4v pv[kScanRows];
#pragma unroll
        for (int i = 0; i < kScanRows; ++i)
          pv[i] = b0 + i < b1
                      ? *reinterpret_cast<const f32x4v*>(blk_P + (int64_t)(b0 + i) * ldn + col)
                      : f32x4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < kScanRows; ++i) ps += pv[i];
      }
    } else {
      for (int b = b0; b < b1; ++b) {
        cs += *reinterpret_cast<const i32x4*>(blk_cnt + (int64_t)b * ldn + col);
        if (blk_P) ps += *reinterpret_cast<const f32x4v*>(blk_P + (int64_t)b * ldn + col);
      }
    }
  }
  i32x4 incl = cs;
  for (int off = 1; off < C; off <<= 1) {
    const i32x4 o = shfl_up4(incl, off, C);
    if (c >= off) incl += o;
  }
  for (int m = C >> 1; m >= 1; m >>= 1) ps += shfl_xor4(ps, m, C);
  const i32x4 pre = incl - cs;  // rows of these experts in earlier chunks
  if (act && c == C - 1) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (col + q < n) s_cnt[col + q] = incl[q];
  }
  if (act && c == 0) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (col + q < n) s_P[col + q] = ps[q];
  }
  __syncthreads();
  int cnt_e = 0;
  if (tid < n) {
    cnt_e = s_cnt[tid];
    if (counts) counts[tid] = cnt_e;
    if (f) f[tid] = (float)((int64_t)cnt_e * n) / (float)((int64_t)k * T);
    if (P && blk_P) P[tid] = s_P[tid] / (float)T;
  }
  const int off_e = scan256(cnt_e, wsum, &s_total);
  if (tid < n) {
    s_off[tid] = off_e;
    offsets[tid] = off_e;
  }
  if (tid == 0) {
    s_off[n] = s_total;
    offsets[n] = s_total;
  }
  if (has_tiles) {
    const int nt_e = tid < n ? (cnt_e + kTileM - 1) / kTileM : 0;
    const int toff = scan256(nt_e, wsum, &s_total);
    if (tid < n) {
      s_toff[tid] = toff;
      tl.off[tid] = toff;
    }
    if (tid == 0) {
      s_toff[n] = s_total;
      tl.off[n] = s_total;
      *tl.count = s_total;
    }
    if (tl.steal && tid < 16) tl.steal[tid] = 0;
  }
  __syncthreads();
  if (has_tiles) {
    // Tile t belongs to the last expert whose first tile is <= t.
    const int total = s_toff[n];
    for (int t = tid; t < total && t < tl.max_tiles; t += kScanThreads) {
      int lo = 0, hi = n;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_toff[mid] <= t)
          lo = mid;
        else
          hi = mid;
      }
      const int r = (t - s_toff[lo]) * kTileM;
      tl.row0[t] = s_off[lo] + r;
      tl.rows[t] = s_cnt[lo] - r < kTileM ? s_cnt[lo] - r : kTileM;
    }
  }
  if (act) {
    i32x4 base;
#pragma unroll
    for (int q = 0; q < 4; ++q) base[q] = (col + q < n ? s_off[col + q] : 0) + pre[q];
    if (cached) {
#pragma unroll
      for (int i = 0; i < kScanRows; ++i) {
        if (b0 + i < b1) *reinterpret_cast<i32x4*>(blk_base + (int64_t)(b0 + i) * ldn + col) = base;
        base += v[i];
      }
    } else {
      for (int b = b0; b < b1; ++b) {
        *reinterpret_cast<i32x4*>(blk_base + (int64_t)b * ldn + col) = base;
        base += *reinterpret_cast<const i32x4*>(blk_cnt + (int64_t)b * ldn + col);
      }
    }
  }
}

// Grouping in one pass of B workgroups, one per route block: every
// workgroup reads the whole [B][ldn] histogram table (small: a few tens of
// KB) in one batch of loads, forms the per-expert totals and its own block's
// prefix, hence the expert offsets and its block's bases, and scatters its
// tokens' (t, j) pairs.  Workgroup b also sums column b of the P partials
// (experts b, b + B, ... when n > B), workgroup 0 writes counts, f and
// offsets, the last workgroup the M-tile list.
// Every workgroup derives the same totals (exact integer sums), so no
// workgroup waits for another.
constexpr int kGroupThreads = 256;
constexpr int kGroupRows = 16;  // table rows a thread has in flight

__global__ __launch_bounds__(kGroupThreads) void group_kernel(
    const int32_t* __restrict__ blk_cnt, const float* __restrict__ blk_P, int B, int64_t T,
    int n, int k, const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ lrank,
    int32_t* __restrict__ counts, float* __restrict__ f, float* __restrict__ P,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm_token,
    int32_t* __restrict__ slot_of, TileList tl) {
  __shared__ int s_tot[kMaxExperts];
  __shared__ int s_base[kMaxExperts];
  __shared__ int s_off[kMaxExperts + 1];
  __shared__ int s_toff[kMaxExperts + 1];
  __shared__ int wsum[4];
  __shared__ int s_total;
  __shared__ float s_red[kGroupThreads / 64];
  const int tid = threadIdx.x, blk = blockIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ldn = blk_ld(n), n4 = ldn >> 2;
  int C = 1;  // row chunks per column: a power of two, n4 * C <= 256
  while (C * 2 * n4 <= kGroupThreads && C * 2 <= 64) C *= 2;
  const int per = (B + C - 1) / C;
  const int e4 = tid / C, c = tid - (tid / C) * C;
  const bool act = e4 < n4;
  const int r0 = c * per < B ? c * per : B;
  const int r1 = r0 + per < B ? r0 + per : B;
  const int64_t col = 4 * e4;
  // This block's first (token, slot) pairs and its first P column are loaded
  // with the table (P rows ascending per thread).
  int e_first = -1, rank_first = 0;
  {
    const int64_t t = (int64_t)blk * kRouteTok + tid / k;
    if (tid < kRouteTok * k && t < T) {
      const int64_t p = t * k + tid % k;
      e_first = topk_idx[p];
      rank_first = lrank[p];
    }
  }
  const bool with_P = blk_P && P && blk < n;
  float p_first = 0.f;
  if (with_P && tid < B) p_first = blk_P[(int64_t)tid * ldn + blk];
  i32x4 tot = {0, 0, 0, 0}, pre = {0, 0, 0, 0};
  if (act) {
    for (int rb = r0; rb < r1; rb += kGroupRows) {
      i32x4 v[kGroupRows];
#pragma unroll
      for (int i = 0; i < kGroupRows; ++i)
        v[i] = rb + i < r1 ? *reinterpret_cast<const i32x4*>(blk_cnt + (int64_t)(rb + i) * ldn + col)
                           : i32x4{0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < kGroupRows; ++i) {
        tot += v[i];
        if (rb + i < blk) pre += v[i];
      }
    }
  }
  for (int m = C >> 1; m >= 1; m >>= 1) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      tot[q] += __shfl_xor(tot[q], m, C);
      pre[q] += __shfl_xor(pre[q], m, C);
    }
  }
  if (act && c == 0) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (col + q < n) {
        s_tot[col + q] = tot[q];
        s_base[col + q] = pre[q];
      }
  }
  // P_e = (column sum of the block partials) / T: a fixed butterfly inside
  // each wave, then the waves in order.
  for (int e = blk; with_P && e < n; e += B) {
    float pacc = e == blk ? p_first : 0.f;
    for (int r = e == blk ? tid + kGroupThreads : tid; r < B; r += kGroupThreads)
      pacc += blk_P[(int64_t)r * ldn + e];
    for (int m = 32; m >= 1; m >>= 1) pacc += __shfl_xor(pacc, m, 64);
    if (lane == 0) s_red[wave] = pacc;
    __syncthreads();
    if (tid == 0) {
      float acc = s_red[0];
#pragma unroll
      for (int w = 1; w < kGroupThreads / 64; ++w) acc += s_red[w];
      P[e] = acc / (float)T;
    }
    __syncthreads();
  }
  __syncthreads();
  const int cnt_e = tid < n ? s_tot[tid] : 0;
  const int off_e = scan256(cnt_e, wsum, &s_total);
  if (tid < n) {
    s_off[tid] = off_e;
    s_base[tid] += off_e;
  }
  if (blk == 0) {
    if (tid < n) {
      offsets[tid] = off_e;
      if (counts) counts[tid] = cnt_e;
      if (f) f[tid] = (float)((int64_t)cnt_e * n) / (float)((int64_t)k * T);
    }
    if (tid == 0) offsets[n] = s_total;
  }
  if (tid == 0) s_off[n] = s_total;
  __syncthreads();
  // This block's (token, slot) pairs.  Ids outside [0, n) and positions
  // outside [0, T*k) break the contract; such slots get slot_of = -1.
  const int64_t R = T * k;
  for (int q = tid; q < kRouteTok * k; q += kGroupThreads) {
    const int64_t t = (int64_t)blk * kRouteTok + q / k;
    if (t >= T) break;
    const int64_t p = t * k + q % k;
    const int e = q == tid ? e_first : topk_idx[p];
    int pos = -1;
    if (e >= 0 && e < n) {
      pos = s_base[e] + (q == tid ? rank_first : lrank[p]);
      if (pos < 0 || pos >= R) pos = -1;
    }
    slot_of[p] = pos;
    if (pos >= 0) perm_token[pos] = (int32_t)t;
  }
  // The M-tile list: the last workgroup (workgroup 0 writes counts, f and
  // offsets).
  if (blk != B - 1 || !tl.off) return;
  emit_tile_list(tl, n, s_tot, s_off, s_toff, wsum, &s_total, kGroupThreads);
}

// ------------------------------------------------ routing of small batches

// Batches of at most 64 tokens (bf16).  The per-block router above puts the
// whole centroid matrix through each of a few CUs and leaves the rest idle;
// here the logits are spread over (token block x 16 experts) workgroups, and
// one workgroup then routes and groups the whole batch, so no per-block
// histograms or bases are needed.

// Logits of 16 tokens x 16 experts (expert group blockIdx.y) into lg[T][n]:
// the same MFMA sequence and reduction as the per-block router, so the
// values are the same bits.
template <bool STAGED>
__global__ __launch_bounds__(kThreads) void logits_small_kernel(
    const uint16_t* __restrict__ u, const uint16_t* __restrict__ cent, int64_t T, int d, int n,
    float* __restrict__ lg) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const RouteSmem s = carve(smem, 16);
  const int64_t blk = blockIdx.x;
  const int e0 = blockIdx.y * 16;
  const int ng = n - e0 < 16 ? n - e0 : 16;
  const uint16_t* cg = cent + (int64_t)e0 * d;
  if constexpr (STAGED)
    logits_bf16_staged<1>(u, cg, T, d, ng, blk, s, smem + route_smem_bytes_aligned(16, 0));
  else
    logits_bf16<1>(u, cg, T, d, ng, blk, s);
  __syncthreads();
  for (int p = threadIdx.x; p < kRouteTok * 16; p += kThreads) {
    const int tl = p >> 4, e = p & 15;
    const int64_t t = blk * kRouteTok + tl;
    if (t < T && e < ng) lg[t * n + e0 + e] = s.lg[tl * s.ldl + e];
  }
}

constexpr int kSmallTok = kSmallBatch;         // tokens one routing workgroup takes
constexpr int kSmallThreads = 16 * kSmallTok;  // a 16-lane DPP row per token

__host__ __device__ inline size_t route_small_smem_bytes(int n, int k) {
  const size_t ldl = (size_t)n + 1;
  return sizeof(float) * 2 * kSmallTok * ldl                          // logits, softmax
         + sizeof(int) * ((size_t)kSmallTok * k + 3 * (kMaxExperts + 1) + 8);
}

// Softmax, top-k, P, counts / f, ranks, offsets, the stable scatter and the
// M-tile list of a batch of T <= 64 tokens, one workgroup: token t is lane
// t of every wave, so one ballot per expert gives its count and the rank of
// each of its tokens.
template <int NB>
__global__ __launch_bounds__(kSmallThreads) void route_small_kernel(
    const float* __restrict__ lg, int64_t T, int n, int k, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_gate, int32_t* __restrict__ counts, float* __restrict__ f,
    float* __restrict__ P, int32_t* __restrict__ offsets, int32_t* __restrict__ perm_token,
    int32_t* __restrict__ slot_of, TileList tl) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int ldl = n + 1;
  float* s_lg = reinterpret_cast<float*>(smem);  // [64][ldl] logits, then ranks
  float* s_sv = s_lg + kSmallTok * ldl;          // [64][ldl] softmax values
  int* s_idx = reinterpret_cast<int*>(s_sv + kSmallTok * ldl);  // [64][k]
  int* s_cnt = s_idx + kSmallTok * k;
  int* s_off = s_cnt + (kMaxExperts + 1);
  int* s_toff = s_off + (kMaxExperts + 1);
  int* wsum = s_toff + (kMaxExperts + 1);
  int* s_total = wsum + 4;
  int* s_rk = reinterpret_cast<int*>(s_lg);
  const int tid = threadIdx.x;
  for (int p = tid; p < T * n; p += kSmallThreads) {
    const int t = p / n;
    s_lg[t * ldl + (p - t * n)] = lg[p];
  }
  __syncthreads();
  {
    const int t = tid >> 4;  // a whole DPP row shares its token
    if (t < T)
      token_topk<NB>(s_lg + t * ldl, s_sv + t * ldl, s_idx + t * k, tid & 15, n, k, true, t,
                     topk_idx, topk_gate);
  }
  __syncthreads();
  // P (waves 0..7): the 8 lanes of a half row take one expert; lane q sums
  // tokens q, q + 8, ... ascending, then a fixed butterfly adds the 8
  // partial sums.  Meanwhile waves 8..15 count and rank.
  constexpr int kHalf = kSmallThreads / 2;
  for (int e0 = tid >> 3; tid < kHalf && e0 < n; e0 += kHalf / 8) {
    const int q = tid & 7;
    float acc = 0.f;
    for (int t = q; t < T; t += 8) acc += s_sv[t * ldl + e0];
    acc += dppf<kQuadX1>(acc);
    acc += dppf<kQuadX2>(acc);
    acc += dppf<kHalfMirror>(acc);
    if (q == 0) P[e0] = acc / (float)T;
  }
  // Counts and ranks: wave 8 + w takes experts w, w + 8, ...; lane = token.
  if (tid >= kHalf) {
    const int lane = tid & 63, wave = (tid - kHalf) >> 6;
    uint64_t bits0 = 0, bits1 = 0, bits2 = 0, bits3 = 0;  // this token's experts
    if (lane < T)
      for (int j = 0; j < k; ++j) {
        const int e = s_idx[lane * k + j];
        const uint64_t b = 1ull << (e & 63);
        const int w = e >> 6;
        bits0 |= w == 0 ? b : 0ull;
        bits1 |= w == 1 ? b : 0ull;
        bits2 |= w == 2 ? b : 0ull;
        bits3 |= w >= 3 ? b : 0ull;
      }
    const uint64_t below = (1ull << lane) - 1ull;
    for (int e = wave; e < n; e += kHalf / 64) {
      const int w = e >> 6;
      const uint64_t word = w == 0 ? bits0 : (w == 1 ? bits1 : (w == 2 ? bits2 : bits3));
      const bool has = (word >> (e & 63)) & 1ull;
      const uint64_t m = __ballot(has);
      if (lane == 0) s_cnt[e] = __popcll(m);
      if (has) s_rk[lane * ldl + e] = __popcll(m & below);
    }
  }
  __syncthreads();
  const int cnt_e = tid < n ? s_cnt[tid] : 0;
  const int off_e = scan256(cnt_e, wsum, s_total);
  if (tid < n) {
    s_off[tid] = off_e;
    offsets[tid] = off_e;
    counts[tid] = cnt_e;
    f[tid] = (float)((int64_t)cnt_e * n) / (float)((int64_t)k * T);
  }
  if (tid == 0) {
    s_off[n] = *s_total;
    offsets[n] = *s_total;
  }
  __syncthreads();
  for (int p = tid; p < T * k; p += kSmallThreads) {
    const int t = p / k;
    const int e = s_idx[p];
    const int pos = s_off[e] + s_rk[t * ldl + e];
    slot_of[p] = pos;
    perm_token[pos] = t;
  }
  if (tl.off) emit_tile_list(tl, n, s_cnt, s_off, s_toff, wsum, s_total, kSmallThreads);
}

// The expert-level balance loss alpha * sum_i f_i P_i ("Expert-level balance
// loss"): the products are formed in parallel into LDS, then one thread adds
// them in ascending i, so the value is that of a plain ascending sum.
__global__ __launch_bounds__(kMaxExperts) void balance_loss_kernel(const float* __restrict__ f,
                                                                   const float* __restrict__ P,
                                                                   int n, float alpha,
                                                                   float* __restrict__ loss) {
  __shared__ __attribute__((aligned(16))) float prod[kMaxExperts];
  const int i = threadIdx.x;
  prod[i] = i < n ? __fmul_rn(f[i], P[i]) : 0.0f;
  __syncthreads();
  if (i == 0) {
    float acc = 0.0f;
    for (int j = 0; j < n; ++j) acc = __fadd_rn(acc, prod[j]);
    loss[0] = __fmul_rn(alpha, acc);
  }
}

constexpr int kTileThreads = 256;

// Offsets that break the documented contract (decreasing, outside
// [0, rows]) are clamped so that every tile stays inside the row range and
// the tile capacity.
__global__ __launch_bounds__(kTileThreads) void tiles_kernel(const int32_t* __restrict__ offsets,
                                                             int G, int64_t rows, TileList tl) {
  __shared__ int wsum[4];
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
  const int toff = scan256(nt_g, wsum, &s_total);
  if (tid < G) {
    tl.off[tid] = toff;
    emit_tiles(tl, toff, first, cnt);
  }
  if (tid == 0) {
    const int total = s_total < tl.max_tiles ? s_total : tl.max_tiles;
    tl.off[G] = total;
    *tl.count = total;
  }
  if (tl.steal && tid < 16) tl.steal[tid] = 0;
}

}  // namespace

hipError_t launch_route(int dtype, const void* u, const void* cent, int64_t T, int d, int n,
                        int k, int32_t* topk_idx, float* topk_gate, int32_t* blk_cnt,
                        float* blk_P, int32_t* lrank, hipStream_t s, float* lg_out, int ld_out) {
  const int B = (int)((T + kRouteTok - 1) / kRouteTok);
  const size_t sm = route_smem_bytes(n, k);
  const int nb = (n + 15) / 16;
  if (dtype == 0) {
#define MOE_ROUTE_F32(NBV)                                                                     \
  {                                                                                            \
    if (sm > kDefaultLds) {                                                                    \
      const hipError_t e = hipFuncSetAttribute((const void*)route_f32_kernel<NBV>,             \
                                               hipFuncAttributeMaxDynamicSharedMemorySize,     \
                                               (int)sm);                                       \
      if (e != hipSuccess) return e;                                                           \
    }                                                                                          \
    hipLaunchKernelGGL(route_f32_kernel<NBV>, dim3(B), dim3(kThreads), sm, s,                  \
                       (const float*)u, (const float*)cent, T, d, n, k, topk_idx, topk_gate,   \
                       blk_cnt, blk_P, lrank);                                                 \
  }
    if (nb <= 1) MOE_ROUTE_F32(1)
    else if (nb <= 2) MOE_ROUTE_F32(2)
    else if (nb <= 4) MOE_ROUTE_F32(4)
    else if (nb <= 8) MOE_ROUTE_F32(8)
    else MOE_ROUTE_F32(16)
#undef MOE_ROUTE_F32
    return hipGetLastError();
  }
#define MOE_ROUTE_CASE(NBV, STG)                                                               \
  {                                                                                            \
    const size_t smv = STG ? route_smem_bytes_aligned(n, k) + (size_t)kWaves * (2 + 2 * NBV) * 1024 \
                           : sm;                                                               \
    if (smv > kDefaultLds) {                                                                   \
      const hipError_t e = hipFuncSetAttribute((const void*)route_bf16_kernel<NBV, STG>,       \
                                               hipFuncAttributeMaxDynamicSharedMemorySize,     \
                                               (int)smv);                                      \
      if (e != hipSuccess) return e;                                                           \
    }                                                                                          \
    hipLaunchKernelGGL((route_bf16_kernel<NBV, STG>), dim3(B), dim3(kThreads), smv, s,         \
                       (const uint16_t*)u, (const uint16_t*)cent, T, d, n, k, topk_idx,        \
                       topk_gate, blk_cnt, blk_P, lrank, lg_out, ld_out);                      \
  }
  // Staged loads while a wave's hidden range fits one round (d <= 2048) and
  // the operand regions fit LDS (n <= 64).
  const bool staged = d <= 2048 && nb <= 4;
  if (nb <= 1) {
    if (staged) MOE_ROUTE_CASE(1, true) else MOE_ROUTE_CASE(1, false)
  } else if (nb <= 2) {
    if (staged) MOE_ROUTE_CASE(2, true) else MOE_ROUTE_CASE(2, false)
  } else if (nb <= 4) {
    if (staged) MOE_ROUTE_CASE(4, true) else MOE_ROUTE_CASE(4, false)
  } else if (nb <= 8) {
    MOE_ROUTE_CASE(8, false)
  } else {
    MOE_ROUTE_CASE(16, false)
  }
#undef MOE_ROUTE_CASE
  return hipGetLastError();
}

bool route_small(int dtype, int64_t T) { return dtype == 1 && T <= kSmallTok; }

hipError_t launch_balance_loss(const float* f, const float* P, int n, float alpha, float* loss,
                               hipStream_t s) {
  hipLaunchKernelGGL(balance_loss_kernel, dim3(1), dim3(kMaxExperts), 0, s, f, P, n, alpha, loss);
  return hipGetLastError();
}

hipError_t launch_logits_small(const void* u, const void* cent, int64_t T, int d, int n, float* lg,
                               hipStream_t s) {
  const int B = (int)((T + kRouteTok - 1) / kRouteTok);
  const dim3 grid((unsigned)B, (unsigned)((n + 15) / 16));
  if (d <= 2048) {
    const size_t sm = route_smem_bytes_aligned(16, 0) + (size_t)kWaves * 4 * 1024;
    hipLaunchKernelGGL(logits_small_kernel<true>, grid, dim3(kThreads), sm, s,
                       (const uint16_t*)u, (const uint16_t*)cent, T, d, n, lg);
  } else {
    hipLaunchKernelGGL(logits_small_kernel<false>, grid, dim3(kThreads),
                       route_smem_bytes(16, 0), s, (const uint16_t*)u, (const uint16_t*)cent, T,
                       d, n, lg);
  }
  return hipGetLastError();
}

hipError_t launch_route_small(const float* lg, int64_t T, int n, int k, int32_t* topk_idx,
                              float* topk_gate, int32_t* counts, float* f, float* P,
                              int32_t* offsets, int32_t* perm_token, int32_t* slot_of,
                              const TileList* tiles, hipStream_t s) {
  hipError_t e = hipSuccess;
  const TileList tl = tiles ? *tiles : TileList{nullptr, nullptr, nullptr, nullptr, 0};
  const size_t sm = route_small_smem_bytes(n, k);
  const int nb = (n + 15) / 16;
#define MOE_ROUTE_SMALL(NBV)                                                                   \
  {                                                                                            \
    if (sm > kDefaultLds) {                                                                    \
      e = hipFuncSetAttribute((const void*)route_small_kernel<NBV>,                            \
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm);            \
      if (e != hipSuccess) return e;                                                           \
    }                                                                                          \
    hipLaunchKernelGGL(route_small_kernel<NBV>, dim3(1), dim3(kSmallThreads), sm, s, lg, T, n, \
                       k, topk_idx, topk_gate, counts, f, P, offsets, perm_token, slot_of, tl); \
  }
  if (nb <= 1) MOE_ROUTE_SMALL(1)
  else if (nb <= 2) MOE_ROUTE_SMALL(2)
  else if (nb <= 4) MOE_ROUTE_SMALL(4)
  else if (nb <= 8) MOE_ROUTE_SMALL(8)
  else MOE_ROUTE_SMALL(16)
#undef MOE_ROUTE_SMALL
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

bool group_in_one_pass(int64_t T, int n) {
  const int64_t B = (T + kRouteTok - 1) / kRouteTok;
  return B * blk_ld(n) <= 32768;  // each workgroup reads the table: at most 128 KB
}

hipError_t launch_group(const int32_t* blk_cnt, const float* blk_P, int64_t T, int n, int k,
                        const int32_t* topk_idx, const int32_t* lrank, int32_t* counts,
                        float* f, float* P, int32_t* offsets, int32_t* perm_token,
                        int32_t* slot_of, const TileList* tiles, hipStream_t s) {
  const int B = (int)((T + kRouteTok - 1) / kRouteTok);
  TileList tl = tiles ? *tiles : TileList{nullptr, nullptr, nullptr, nullptr, 0};
  hipLaunchKernelGGL(group_kernel, dim3(B), dim3(kGroupThreads), 0, s, blk_cnt, blk_P, B, T, n,
                     k, topk_idx, lrank, counts, f, P, offsets, perm_token, slot_of, tl);
  return hipGetLastError();
}

hipError_t launch_tiles(const int32_t* offsets, int n_groups, int64_t rows,
                        const TileList& tiles, hipStream_t s) {
  hipLaunchKernelGGL(tiles_kernel, dim3(1), dim3(kTileThreads), 0, s, offsets, n_groups, rows,
                     tiles);
  return hipGetLastError();
}

}  // namespace moe
