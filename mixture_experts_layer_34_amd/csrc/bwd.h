// Host-side launchers of the backward pass's kernels (internal to libmoe.so).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// One product of the backward pass, C = A B over bf16 operands with fp32
// accumulation, in one of two groupings:
//   rows  - C's rows are grouped rows (a tile list or `rows` rows of one
//           group); group e multiplies by its own B (B + e * b_gstride);
//           K is fixed.
//   k     - every group g owns a K range (memory rows koff[g] .. koff[g+1]-1,
//           or g*kchunk .. min((g+1)*kchunk, K) when koff is null) and writes
//           its own M x N output at C + g * c_gstride (weight gradients,
//           partial sums over token chunks).
// Operands live in memory either K-contiguous (element (i, k) at
// p[i * ld + k]) or K-strided (element (i, k) at p[k * ld + i]); rows taken
// in another order are gathered beforehand.  Pass p (npass = 1 or 2)
// uses A[p] and B[p]; a second pass adds A[1] B[1] into the same
// accumulators (dx = da W1 + db W3).
struct BgSeg {
  const void* A[2];
  int64_t lda;
  const void* B[2];
  int64_t ldb;
  const void* B2;        // second B of the dual product (a and b of the SwiGLU)
  int64_t b_gstride;     // rows grouping: elements between groups' B
  int npass;
  int M, N, K;           // k grouping: output M x N per group; rows: N, K
  int a_lim, b_lim;      // valid elements along the strided side of A / B
                         // (multiples of 8; the memory rows hold at least as many)
  int bk_lim;            // rows grouping: K rows of B that exist (K-strided B)
  int64_t rows;          // rows grouping without a tile list
  const int32_t* t_row0;  // tile list (rows grouping), nullable
  const int32_t* t_rows;
  const int32_t* t_off;
  const int32_t* t_count;
  int n_groups;
  int max_tiles;
  const int32_t* koff;   // k grouping
  int kchunk;
  int G;
  void* C;
  int64_t ldc;
  int64_t c_gstride;
  int c_stream;          // k grouping: C is a final result no later kernel of the
                         // call reads: stored non-temporal, so it does not evict
                         // the operands the other tiles share in L2
  // SwiGLU-backward epilogue (rows grouping, dual product): q, da, db, gh
  // share C's row pitch ldc.
  const void* q;
  const float* gate;  // per grouped row; null: weight one and no dgp
  void* da;
  void* db;
  void* gh;
  float* dgp;
  int ldgp;
  // du epilogue: C[t] = acc + resid[t] + dxs[t] + sum_j dxp[slot_of[t][j]]
  const void* resid;
  const void* dxs;
  const void* dxp;
  const int32_t* slot_of;
  int k;
};

constexpr int kBgMaxSeg = 8;
// Bytes of one BG_WGRAD output group (M * ldc * 4) must stay below this: the
// epilogue stores through a buffer resource and drops offsets at or past it.
constexpr int kBwdOutBytes = 0x7ffffff0;
constexpr int kBgTile = 128;  // rows and columns of a rows-grouping tile
constexpr int kBgK = 64;      // K slice

enum BgKind {
  BG_LOGITS = 0,  // rows, K-contiguous B, fp32 out
  BG_PROJ = 1,    // rows, K-strided B, bf16 out (q = dh W2, dx = da W1 + db W3)
  BG_SWIGLU = 2,  // rows, K-contiguous dual B, SwiGLU-backward epilogue
  BG_DU = 3,      // rows, K-strided B, du epilogue
  BG_WGRAD = 4,   // k grouping, both operands K-strided, fp32 out, 256 x 128 tiles
  BG_PROJ_PACKED = 5,   // BG_PROJ with B in the packed weight layout (row length ldb)
  BG_SWIGLU_PACKED = 6  // BG_SWIGLU with B and B2 packed
};

// BG_WGRAD takes work_ctr: kWgQueues ints in device memory, zero when the
// launch starts (the workgroups' tile queues; they are left nonzero).
constexpr int kWgQueues = 8;
hipError_t launch_bg(BgKind kind, const BgSeg* segs, int nseg, hipStream_t s,
                     int* work_ctr = nullptr);

// Rows of u and dh in grouped order and the gate of each grouped row:
// xp[slot_of[t][j]] = u[t], dhp[slot_of[t][j]] = dh[t],
// gperm[slot_of[t][j]] = topk_gate[t][j]  (bf16 rows of d elements); also
// zeroes clear[0 .. kWgQueues-1] when clear is not null (a later BG_WGRAD
// launch's queues).
hipError_t launch_gather_rows(const int32_t* slot_of, const float* topk_gate, const void* u,
                              const void* dh, int64_t T, int k, int d, void* xp, void* dhp,
                              float* gperm, int* clear, hipStream_t s);

// SwiGLU backward from kept pre-activations pre [rows][2F] (a = W1 x in
// columns 0..F-1, b = W3 x in F..2F-1, bf16) and q [rows][F] (bf16):
// da = g q b SiLU'(a), db = g q SiLU(a), gh = g SiLU(a) b (bf16 [rows][F]),
// g = gate[row] (null: 1).  With dgp: per-row partial sums of <q, SiLU(a) b>
// over 64-column blocks, dgp [rows][ldgp] (blocks beyond F written zero).
// Rows at or beyond *nrows (when nrows is not null) are left alone.
hipError_t launch_swiglu_bwd(const uint16_t* q, const uint16_t* pre, const float* gate,
                             const int32_t* nrows, int64_t rows, int F, uint16_t* da,
                             uint16_t* db, uint16_t* gh, float* dgp, int ldgp, hipStream_t s);

// Per token: softmax of the logits lg [T][ldlg] (fp32), the gate gradients
// sum_p dgp[slot][p], the balance term alpha f_i / T, and the softmax
// backward dl = s (ds - <s, ds>) into dl [T][ldl] (bf16, zero padded).
hipError_t launch_softmax_bwd(const float* lg, int ldlg, int ldl, int64_t T, int n, int k,
                              const int32_t* topk_idx, const int32_t* slot_of, const float* dgp,
                              int ldgp, const float* f, float alpha, uint16_t* dl, hipStream_t s);

// out[i] = sum_g slabs[g * count + i]   (count a multiple of 4)
hipError_t launch_slab_sum(const float* slabs, int G, int64_t count, float* out, hipStream_t s);

}  // namespace moe
