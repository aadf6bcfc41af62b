// Grouped SwiGLU FFN for groups of few rows: the decode regime of the
// DeepSeekMoE layer (tens of tokens, so every routed expert sees a handful
// of rows).  There the work is streaming every expert's weights once from
// HBM; the 128-row tiles of the main grouped GEMM would spend their time on
// padding.
//
// A work item is one wave (a workgroup of its own: there is no LDS and no
// barrier, and single waves spread evenly over the CUs).  It owns 32-row
// bands of packed weights (up: the W1 and the W3 band of the same 32 d_ff
// columns; down: one band of W2) and the group's rows in passes of 32 (one
// pass unless a group holds more than 32 rows; a lone dense group, the
// shared experts, gives each pass an item of its own so its waves end with
// the others).  The MFMA 32x32x16 takes a weight band as its first operand
// and 32 activation rows as its second; 16-wide k blocks are kept in flight
// in a register ring.  SwiGLU is applied in registers (gate and up values
// of one (row, column) sit in the same lane and register).
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kSkThreads = 64;  // one wave
// 16-wide k blocks in flight per wave: 6 for a band pair, 12 for a single
// band, 12 KB of weights either way.  Both fit 168 registers, so three waves
// share a SIMD (a 64-token layer's 2992 up-projection items then all run in
// one round; eight blocks per band pair would not fit and left a second
// round of a few waves).
constexpr int kSkDepth = 6;
constexpr int kSkWavesPerSimd = 3;
template <bool TWO>
constexpr int sk_depth() {
  return TWO ? kSkDepth : 2 * kSkDepth;
}

typedef __bf16 bf16x4s __attribute__((ext_vector_type(4)));

struct SkSeg {
  const uint16_t* X;       // activations
  const int32_t* x_rows;   // nullable: row of X for each grouped row
  int64_t ldx;
  const uint16_t* W0;      // packed; up: W1, down: W2
  const uint16_t* W1;      // packed; up: W3
  int64_t w_stride;        // elements per group
  int K;                   // reduction length (multiple of 32)
  int N;                   // output columns per group (multiple of 32)
  uint16_t* C;
  int64_t ldc;
  const int32_t* offsets;  // nullable: a single group of `rows` rows
  int n_groups;
  int64_t rows;
  int nbands;              // band items per group
  int passes;              // single group: 32-row passes split over items (else 1)
  int nblk;                // items per group
};

struct SkArgs {
  SkSeg seg[2];  // seg[0] is dealt first
  int nseg;
};

// All passes of one item over its group's rows.  TWO: a second weight band
// (the up projection's W3 band) is streamed next to the first.  The first
// ring of weight blocks depends only on the item's expert and band, so it is
// requested before the group's rows are read (offs: the groups' row offsets,
// nullable for a fixed r0 / nrows): the weight stream does not wait for the
// offsets -> row map -> activation chain.
template <bool UP, bool TWO>
__device__ __forceinline__ void skinny_item(const SkSeg& g, const int32_t* offs, int e, int64_t r0,
                                            int64_t nrows, const uint16_t* wa, const uint16_t* wb,
                                            int row_a, int row_b) {
  const int lane = threadIdx.x;
  const int KB = g.K / 16;
  const uint32_t wl = (uint32_t)lane * 16u;  // this lane's bytes in a 1 KB k block
  const int tok = lane & 31;                 // activation row of this lane in a pass
  const int kq = (lane >> 5) * 8;            // its k sub-offset in a 16-wide block
  constexpr int kDepth = sk_depth<TWO>();
  bf16x8 fa[kDepth], fb[TWO ? kDepth : 1], fx[kDepth];
  auto wload = [&](int slot, int kb) {
    kb = kb < KB ? kb : KB - 1;  // past the end: a block nobody reads
    fa[slot] = ld_off<bf16x8>(wa, wl + (uint32_t)kb * 1024u);
    if constexpr (TWO) fb[slot] = ld_off<bf16x8>(wb, wl + (uint32_t)kb * 1024u);
  };
#pragma unroll
  for (int j = 0; j < kDepth; ++j) wload(j, j);
  if (offs) {  // caller data: clamped into [0, rows]
    int64_t a = offs[e], b = offs[e + 1];
    a = a < 0 ? 0 : (a > g.rows ? g.rows : a);
    b = b < a ? a : (b > g.rows ? g.rows : b);
    r0 = a;
    nrows = b - a;
  }
  // An expert nobody chose: its weights are not read past the first ring,
  // whose values go unused.
  if (nrows <= 0) return;

  for (int64_t p0 = 0; p0 < nrows; p0 += 32) {
    int64_t pr = p0 + tok;
    if (pr > nrows - 1) pr = nrows - 1;  // padding lanes repeat the last row
    const int64_t xr = g.x_rows ? (int64_t)g.x_rows[r0 + pr] : r0 + pr;
    // 32-bit byte offset from the uniform base (operands stay below 2^31
    // elements)
    const uint32_t xo = (uint32_t)(xr * g.ldx + kq) * 2u;

    f32x16 acc_a, acc_b;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      acc_a[j] = 0.f;
      acc_b[j] = 0.f;
    }
    auto xload = [&](int slot, int kb) {
      kb = kb < KB ? kb : KB - 1;
      fx[slot] = ld_off<bf16x8>(g.X, xo + (uint32_t)kb * 32u);
    };
    auto load = [&](int slot, int kb) {
      wload(slot, kb);
      xload(slot, kb);
    };
    auto mma = [&](int slot) {
      acc_a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[slot], fx[slot], acc_a, 0, 0, 0);
      if constexpr (TWO)
        acc_b = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[slot], fx[slot], acc_b, 0, 0, 0);
    };
    if (p0 > 0) {  // a further pass streams the band again
#pragma unroll
      for (int j = 0; j < kDepth; ++j) wload(j, j);
    }
#pragma unroll
    for (int j = 0; j < kDepth; ++j) xload(j, j);
    int kb0 = 0;
    for (; kb0 + kDepth <= KB; kb0 += kDepth) {
#pragma unroll
      for (int j = 0; j < kDepth; ++j) {
        mma(j);
        load(j, kb0 + j + kDepth);
      }
    }
#pragma unroll
    for (int j = 0; j < kDepth; ++j)
      if (kb0 + j < KB) mma(j);

    // Lane: activation row tok of this pass; register r: band row
    // 8*(r/4) + 4*(lane/32) + r%4.  Four consecutive columns per group of
    // four registers leave as one 8-byte store.
    if (p0 + tok < nrows) {
      uint16_t* crow = g.C + (r0 + p0 + tok) * g.ldc;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int cofs = 8 * q + 4 * (lane >> 5);
        float va[4], vb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          va[i] = acc_a[4 * q + i];
          vb[i] = acc_b[4 * q + i];
        }
        if (UP) {
          float h[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) h[i] = silu(va[i]) * vb[i];
          *reinterpret_cast<bf16x4s*>(crow + row_a + cofs) =
              bf16x4s{(__bf16)h[0], (__bf16)h[1], (__bf16)h[2], (__bf16)h[3]};
        } else {
          *reinterpret_cast<bf16x4s*>(crow + row_a + cofs) =
              bf16x4s{(__bf16)va[0], (__bf16)va[1], (__bf16)va[2], (__bf16)va[3]};
          if (TWO)
            *reinterpret_cast<bf16x4s*>(crow + row_b + cofs) =
                bf16x4s{(__bf16)vb[0], (__bf16)vb[1], (__bf16)vb[2], (__bf16)vb[3]};
        }
      }
    }
  }
}

template <bool UP>
__global__ __launch_bounds__(kSkThreads, kSkWavesPerSimd) void skinny_kernel(SkArgs args) {
  int L = blockIdx.x;
  const int G0 = args.seg[0].n_groups * args.seg[0].nblk;
  const int si = L < G0 ? 0 : 1;
  if (si) L -= G0;
  const SkSeg& g = args.seg[si];
  const int e = L / g.nblk;
  int blk = L - e * g.nblk;
  int64_t r0 = 0, nrows = g.rows;
  if (!g.offsets && g.passes > 1) {
    // Runs of 8 * passes items: 8 bands x passes row passes, the passes of
    // one band 8 items apart so they are dispatched to the same XCD and
    // share its L2 for the band's weights.
    const int run = 8 * g.passes, q = blk % run, pass = q / 8;
    blk = (blk / run) * 8 + (q & 7);
    if (blk >= g.nbands) return;
    r0 = (int64_t)pass * 32;
    nrows = g.rows - r0 < 32 ? g.rows - r0 : 32;
  }
  const int KB = g.K / 16;
  const uint16_t* base = g.W0 + (int64_t)e * g.w_stride;
  if (UP) {
    const int row = blk * 32;  // W1 rows == W3 rows
    if (row >= g.N) return;
    const int64_t bo = (int64_t)(row >> 5) * KB * 512;
    skinny_item<true, true>(g, g.offsets, e, r0, nrows, base + bo,
                            g.W1 + (int64_t)e * g.w_stride + bo, row, row);
  } else {
    const int row = blk * 32;
    if (row >= g.N) return;
    const uint16_t* wa = base + (int64_t)(row >> 5) * KB * 512;
    skinny_item<false, false>(g, g.offsets, e, r0, nrows, wa, wa, row, row);
  }
}

SkSeg sk_seg(const FfnArgs& a, bool up) {
  SkSeg s{};
  if (up) {
    s.X = (const uint16_t*)a.x;
    s.x_rows = a.x_rows;
    s.ldx = a.ldx;
    s.W0 = (const uint16_t*)a.w1;
    s.W1 = (const uint16_t*)a.w3;
    s.w_stride = (int64_t)a.d_ff_g * a.d;
    s.K = a.d;
    s.N = a.d_ff_g;
    s.C = (uint16_t*)a.hbuf;
    s.ldc = a.d_ff_g;
    s.nblk = (a.d_ff_g + 31) / 32;
  } else {
    s.X = (const uint16_t*)a.hbuf;
    s.x_rows = nullptr;
    s.ldx = a.d_ff_g;
    s.W0 = (const uint16_t*)a.w2;
    s.W1 = nullptr;
    s.w_stride = (int64_t)a.d * a.d_ff_g;
    s.K = a.d_ff_g;
    s.N = a.d;
    s.C = (uint16_t*)a.y;
    s.ldc = a.d;
    s.nblk = (a.d + 31) / 32;
  }
  s.offsets = a.tiles ? a.offsets : nullptr;
  s.n_groups = a.tiles ? a.n_groups : 1;
  s.rows = a.rows;
  // A single group's 32-row passes go to separate items, so its waves take
  // as long as the others' instead of a multiple.
  s.nbands = s.nblk;
  s.passes = 1;
  if (!s.offsets && s.rows > 32) {
    s.passes = (int)((s.rows + 31) / 32);
    s.nblk = (s.nbands + 7) / 8 * 8 * s.passes;
  }
  return s;
}

}  // namespace

hipError_t launch_ffn_skinny(const FfnArgs* segs, int nseg, bool up, hipStream_t s) {
  // An item streams one band pair (up) or one band (down) over the whole
  // reduction; the segment with the longer reduction is dealt first.
  int order[2] = {0, 1};
  if (nseg == 2 && segs[1].d_ff_g > segs[0].d_ff_g) {
    order[0] = 1;
    order[1] = 0;
  }
  SkArgs args{};
  int grid = 0;
  for (int oi = 0; oi < nseg; ++oi) {
    const FfnArgs& a = segs[order[oi]];
    if (a.rows == 0) continue;
    args.seg[args.nseg] = sk_seg(a, up);
    grid += args.seg[args.nseg].n_groups * args.seg[args.nseg].nblk;
    ++args.nseg;
  }
  if (args.nseg == 0) return hipSuccess;
  if (up)
    hipLaunchKernelGGL(skinny_kernel<true>, dim3((unsigned)grid), dim3(kSkThreads), 0, s, args);
  else
    hipLaunchKernelGGL(skinny_kernel<false>, dim3((unsigned)grid), dim3(kSkThreads), 0, s, args);
  return hipGetLastError();
}

}  // namespace moe
