// Host-side launchers of the gfx950 kernels (internal to libmoe.so).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kRouteTok = 16;   // tokens per route block (one ballot histogram each)
constexpr int kTileM = 128;     // rows per grouped-GEMM M-tile
constexpr int kMaxExperts = 256;

// Row pitch (elements) of the per-route-block arrays (block histograms,
// P partials, per-block bases): n rounded up to 4 so rows hold whole
// 16-byte vectors; the padding columns hold zeros.
__host__ __device__ inline int blk_ld(int n) { return (n + 3) & ~3; }

// Device tile list of a grouped problem (built by the scan / tile kernels).
struct TileList {
  int32_t* row0;    // [max_tiles] first grouped row of each M-tile
  int32_t* rows;    // [max_tiles] rows in the tile (1..kTileM)
  int32_t* off;     // [n_groups+1] first M-tile of each group
  int32_t* count;   // [1] number of M-tiles
  int max_tiles;    // capacity (host bound)
  // nullable: [16] per-XCD claim counters of the up (0..7) and down (8..15)
  // projections' launch tails, zeroed by the kernel that writes the list
  int32_t* steal = nullptr;
};

// Router: logits, softmax, top-k, per-block P partial sums, per-block
// histogram and per-(token, slot) rank inside its block.  bf16 with lg_out:
// also the fp32 logits, lg_out [T][ld_out] (ld_out >= n, zero padded).
hipError_t launch_route(int dtype, const void* u, const void* cent, int64_t T, int d, int n,
                        int k, int32_t* topk_idx, float* topk_gate, int32_t* blk_cnt,
                        float* blk_P, int32_t* lrank, hipStream_t s, float* lg_out = nullptr,
                        int ld_out = 0);

// Routing and grouping of batches of at most 64 tokens (bf16) in two
// launches: logits over (token block x 16 experts) workgroups into lg
// [T][n] fp32, then one workgroup for softmax, top-k, counts, f, P, offsets,
// perm_token, slot_of and the tile list (when tiles != nullptr).
constexpr int kSmallBatch = 64;  // most tokens of the small-batch routing
bool route_small(int dtype, int64_t T);
hipError_t launch_logits_small(const void* u, const void* cent, int64_t T, int d, int n, float* lg,
                               hipStream_t s);
hipError_t launch_route_small(const float* lg, int64_t T, int n, int k, int32_t* topk_idx,
                              float* topk_gate, int32_t* counts, float* f, float* P,
                              int32_t* offsets, int32_t* perm_token, int32_t* slot_of,
                              const TileList* tiles, hipStream_t s);

// loss[0] = alpha * sum_{i < n} f_i P_i, ascending i (n <= kMaxExperts).
hipError_t launch_balance_loss(const float* f, const float* P, int n, float alpha, float* loss,
                               hipStream_t s);

// Histogram and ranks from a given topk_idx (standalone grouping).
hipError_t launch_hist(const int32_t* topk_idx, int64_t T, int n, int k, int32_t* blk_cnt,
                       int32_t* lrank, hipStream_t s);

// Column scan of the block histograms: counts, f, P (when blk_P), offsets,
// per-block bases, and the M-tile list (when tiles != nullptr).
hipError_t launch_scan(const int32_t* blk_cnt, const float* blk_P, int64_t T, int n, int k,
                       int32_t* counts, float* f, float* P, int32_t* offsets,
                       int32_t* blk_base, const TileList* tiles, hipStream_t s);

// Scan and scatter in one pass of one workgroup per route block, for tables
// small enough that every workgroup reads all of it (group_in_one_pass).
bool group_in_one_pass(int64_t T, int n);
hipError_t launch_group(const int32_t* blk_cnt, const float* blk_P, int64_t T, int n, int k,
                        const int32_t* topk_idx, const int32_t* lrank, int32_t* counts,
                        float* f, float* P, int32_t* offsets, int32_t* perm_token,
                        int32_t* slot_of, const TileList* tiles, hipStream_t s);

// Scatter to grouped order (+ optional row gather of u into x_perm).
hipError_t launch_scatter(const int32_t* topk_idx, const int32_t* lrank,
                          const int32_t* blk_base, int64_t T, int n, int k,
                          int32_t* perm_token, int32_t* slot_of, const void* u, void* x_perm,
                          int row_bytes, hipStream_t s);

// M-tile list from device offsets (standalone grouped FFN).
hipError_t launch_tiles(const int32_t* offsets, int n_groups, int64_t rows,
                        const TileList& tiles, hipStream_t s);

struct FfnArgs {
  int dtype;
  const void* x;           // activations
  const int32_t* x_rows;   // nullable: source row of x for each grouped row
  int64_t ldx;             // row stride of x (elements)
  const void* w1;          // [G][d_ff_g][d]
  const void* w3;
  const void* w2;          // [G][d][d_ff_g]
  int n_groups;
  int d;
  int d_ff_g;
  int64_t rows;            // total grouped rows
  const int32_t* offsets;  // [G+1] device (fp32 path and tile-less launches use it)
  const TileList* tiles;   // nullptr: single group of `rows` rows
  void* hbuf;              // [rows][d_ff_g] intermediate
  void* y;                 // [rows][d]
  bool packed;             // weights in the packed layout (bf16 only)
  void* preact;            // nullable: [rows][2 d_ff_g] bf16 W1 x | W3 x kept for the
                           // backward (tiled bf16 up projection only)
};

// Packs a [rows][K] bf16 matrix (rows % 32 == 0, K % 16 == 0) into the
// MFMA-block layout the packed grouped FFN reads.
hipError_t launch_pack(const void* src, void* dst, int64_t rows, int K, hipStream_t s);
hipError_t launch_grouped_ffn(const FfnArgs& a, hipStream_t s);  // up then down
// One launch over 1 or 2 segments (e.g. routed experts and shared experts).
hipError_t launch_ffn_up(const FfnArgs* segs, int nseg, hipStream_t s);    // hbuf = SwiGLU(x W1, x W3)
hipError_t launch_ffn_down(const FfnArgs* segs, int nseg, hipStream_t s);  // y = hbuf W2
// Same two projections for groups of few rows (packed bf16 weights only):
// weight streaming with no row tiles; any row count is correct, more than
// 32 rows in a group re-stream its weights per 32 rows.
hipError_t launch_ffn_skinny(const FfnArgs* segs, int nseg, bool up, hipStream_t s);

hipError_t launch_combine(int dtype, const void* residual, const void* shared_out,
                          const void* y_perm, const int32_t* slot_of, const float* gate,
                          void* h, int64_t T, int d, int k, hipStream_t s);

}  // namespace moe
