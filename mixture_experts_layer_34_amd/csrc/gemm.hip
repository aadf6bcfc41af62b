// Grouped SwiGLU FFN: for each group (expert) g and its rows X_g,
//   H_g = SiLU(X_g W1_g^T) * (X_g W3_g^T)      (up + SwiGLU, rounded to bf16)
//   Y_g = H_g W2_g^T                           (down)
// The expert FFN is SwiGLU ("GLU Variants Improve Transformer", cited by the
// DeepSeekMoE card); grouping tokens per expert and fusing the weight
// matrices is the page's note on production layers.
//
// bf16 path.  A workgroup of 4 waves computes a 128-row tile; each wave
// owns all 128 rows and NBW 32-column weight bands as 4 x NBW MFMA 32x32x16
// blocks (fp32 accumulators).  Packed weights (the fast path, PipePacked):
// NBW = 2, 128 x 256 tiles, two workgroups per CU, each wave streaming its
// weight fragments straight into registers while the activations go
// through LDS.  Row-major weights (PipeLds): NBW = 4, 128 x 512 tiles, one
// workgroup per CU, both operands staged through LDS.  K advances in 32-wide
// slices through a software pipeline whose loads, LDS traffic and MFMAs are
// interleaved one MFMA at a time so the memory system and the matrix cores
// work concurrently.
// For the up projection a wave's columns are bands of W1 followed by the
// same bands of W3, so gate and up values of one output land in the same
// lane and the SwiGLU is applied in registers.  The MFMAs take the
// weights as their first operand, so each accumulator holds the transposed
// block: a lane owns one token and four consecutive output columns per
// register group, which leave as one packed 8-byte LDS write, then through
// the staging tile as coalesced 16-byte stores.
// One launch can hold two segments (routed experts from a device tile list,
// then the shared experts as one group) so both fill the GPU together; no
// host synchronisation is needed and workgroups beyond the live tile count
// exit.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int BM = kTileM;          // 128 rows (tokens)
constexpr int BK = 32;              // K slice
constexpr int LDK = BK + 8;         // padded LDS row (elements): 80 B
constexpr int kThreads = 256;

// Tile width: NBW 32-row weight bands per wave, 4 waves.  NBW = 4 gives
// 128 x 512 tiles (one workgroup per CU); NBW = 2 gives 128 x 256 tiles
// with half the accumulators, so two workgroups share a CU and one's
// prologue and epilogue overlap the other's MFMAs.
template <int NBW>
struct Tile {
  static constexpr int WN = 32 * NBW;  // weight rows per wave
  static constexpr int BN = 4 * WN;    // weight rows per tile
  static constexpr int UPC = BN / 2;   // d_ff columns per up tile (W1 + W3 rows)
};
constexpr int BN = Tile<4>::BN;       // the row-major-weight pipeline's tile
constexpr int kUpCols = Tile<4>::UPC;

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

struct GemmSeg {
  const uint16_t* A;
  const int32_t* a_rows;  // nullable gather map
  int64_t lda;
  const uint16_t* B0;     // up: W1, down: W2
  const uint16_t* B1;     // up: W3
  int64_t b_stride;       // elements per group
  int K;
  int N;                  // output columns per group
  uint16_t* C;
  int64_t ldc;
  uint16_t* P;            // up, nullable: pre-activations [rows][2N] (W1 x | W3 x)
  int nN;                 // column tiles
  const int32_t* tile_row0;
  const int32_t* tile_rows;
  const int32_t* tile_off;  // nullable: single group of single_rows rows
  const int32_t* num_tiles;
  int n_groups;
  int64_t single_rows;
};

struct GemmArgs {
  GemmSeg seg[2];
  int nseg;
  int32_t* steal;  // nullable: [8] per-XCD claim counters, zero at launch
};

// Launch tail.  Workgroup w runs on XCD w % 8 and xcd_remap2 gives each XCD
// a contiguous run of tiles; the XCDs' finishing times still spread by
// several percent.  With claim counters, the last eighth of each XCD's run
// (routed tiles only: the shared ones are dealt first) is handed out by an
// atomic per XCD: its own workgroups claim from it first, and workgroups
// with no tile of their own (the grid is sized for the largest possible
// tile list) and those whose XCD ran dry claim from the XCD with the most
// left.  Every claimable tile has at least one claimer on its own XCD and
// each claim index is unique, so every tile runs exactly once; nothing
// waits on another workgroup.
__device__ __forceinline__ int xcd_items(int G, int x) { return G / 8 + (x < G % 8 ? 1 : 0); }

__device__ __forceinline__ int xcd_claimable(int G, int G1, int x) {
  const int q = xcd_items(G, x), q0 = q - xcd_items(G1, x);
  const int c = q >> 3;
  return c < q0 ? c : q0;
}

// The workgroup slot this workgroup runs (a workgroup index in the static
// deal), or -1: none left.
__device__ int claim_tile(int w, int G, int G1, int32_t* steal) {
  __shared__ int s_claim;
  const int x = w & 7, i = w >> 3;
  const int q = xcd_items(G, x), sn = xcd_claimable(G, G1, x);
  if (i < q - sn) return w;  // the static part of this XCD's run
  if (threadIdx.x == 0) {
    int got = -1;
    if (i < q) {  // own claim first
      const int c = __hip_atomic_fetch_add(&steal[x], 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
      if (c < sn) got = 8 * (q - sn + c) + x;
    }
    for (int attempt = 0; got < 0 && attempt < 3; ++attempt) {
      int cnt[8];  // all eight counters in flight at once
#pragma unroll
      for (int y = 0; y < 8; ++y)
        cnt[y] = __hip_atomic_load(&steal[y], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      int best = -1, left = 0;
#pragma unroll
      for (int y = 0; y < 8; ++y) {
        const int l = xcd_claimable(G, G1, y) - cnt[y];
        if (l > left) {
          left = l;
          best = y;
        }
      }
      if (best < 0) break;
      const int c = __hip_atomic_fetch_add(&steal[best], 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
      const int sy = xcd_claimable(G, G1, best);
      if (c < sy) got = 8 * (xcd_items(G, best) - sy + c) + best;
    }
    s_claim = got;
  }
  __syncthreads();
  return s_claim;
}

// Weight packing: [rows][K] row-major -> 32-row bands, each a run of 16-wide
// k blocks of 512 elements in MFMA operand order (lane l holds row l % 32,
// k 8*(l/32) .. +8 of the block).  One thread moves one 16-byte chunk.
__global__ __launch_bounds__(256) void pack_kernel(const uint16_t* __restrict__ src,
                                                   uint16_t* __restrict__ dst, int64_t rows,
                                                   int K) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t kc_per_row = K / 8;
  if (c >= rows * kc_per_row) return;
  const int64_t row = c / kc_per_row;
  const int kc = (int)(c - row * kc_per_row);
  const int64_t band = row >> 5;
  const int r = (int)(row & 31);
  const int kb = kc >> 1, h = kc & 1;
  const int64_t o = ((band * (K / 16) + kb) * 64 + (r + 32 * h)) * 8;
  *reinterpret_cast<u32x4*>(dst + o) = *reinterpret_cast<const u32x4*>(src + row * K + kc * 8);
}

__device__ __forceinline__ int seg_m_tiles(const GemmSeg& g) {
  return g.tile_off ? *g.num_tiles : (int)((g.single_rows + BM - 1) / BM);
}

struct Stage {
  u32x4 a[2], b[8];
};
template <int MB>
struct Frag {
  bf16x8 a[2][MB], b[2][4];
};

// Weights row-major: both operands staged through LDS.
template <bool UP, int MB>
struct PipeLds {
  const GemmSeg& g;
  const uint16_t* b0base;
  const uint16_t* b1base;
  uint32_t aoff[2], boff[8];
  int ns, nr, lane, lc, lr;
  uint16_t (*sA)[BM * LDK];
  uint16_t (*sB)[BN * LDK];

  // Slices past the end are clamped to the last one, so the pipeline body
  // has no branches; those extra loads land in a buffer nobody reads.
  __device__ __forceinline__ void gload(Stage& st, int s) const {
    s = s < ns ? s : ns - 1;
    const uint32_t k0 = (uint32_t)s * (BK * 2);
#pragma unroll
    for (int i = 0; i < 2; ++i) st.a[i] = ld_off<u32x4>(g.A, aoff[i] + k0);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      st.b[i] = ld_off<u32x4>((UP && i >= 4) ? b1base : b0base, boff[i] + k0);
  }
  __device__ __forceinline__ void sstore(const Stage& st, int buf) const {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      *reinterpret_cast<u32x4*>(&sA[buf][(lr + 64 * i) * LDK + lc * 8]) = st.a[i];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *reinterpret_cast<u32x4*>(&sB[buf][(lr + 64 * i) * LDK + lc * 8]) = st.b[i];
  }
  __device__ __forceinline__ void rfrag(Frag<MB>& f, int buf) const {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int ko = kk * 16 + (lane >> 5) * 8;
#pragma unroll
      for (int mi = 0; mi < MB; ++mi)
        f.a[kk][mi] =
            *reinterpret_cast<const bf16x8*>(&sA[buf][(mi * 32 + (lane & 31)) * LDK + ko]);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int brow = UP ? ((nb >> 1) * kUpCols + nr + (nb & 1) * 32) : nr + nb * 32;
        f.b[kk][nb] = *reinterpret_cast<const bf16x8*>(&sB[buf][(brow + (lane & 31)) * LDK + ko]);
      }
    }
  }
  __device__ __forceinline__ void mma(const Frag<MB>& f, f32x16 (&acc)[4][4]) const {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int mi = 0; mi < MB; ++mi)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          acc[mi][nb] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[kk][nb], f.a[kk][mi], acc[mi][nb], 0, 0, 0);
  }
  // One MFMA at a time, interleaved with the fragment reads of the next
  // slice, then the LDS writes and global loads of later slices.
  __device__ __forceinline__ static void schedule() {
    constexpr int nm = 8 * MB, nrd = 2 * (MB + 4);
#pragma unroll
    for (int i = 0; i < nm; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      if (i < nrd) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
      if (i >= nm - 12 && i < nm - 2) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // DS write
      if (i >= nm - 10) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
    }
  }
  __device__ __forceinline__ void run(f32x16 (&acc)[4][4]) const {
    Stage R;
    Frag<MB> F0, F1;
    gload(R, 0);
    sstore(R, 0);
    gload(R, 1);
    sstore(R, 1);
    __syncthreads();
    rfrag(F0, 0);
    gload(R, 2);
    int s = 0;
    for (; s + 2 <= ns; s += 2) {
      // F0 = slice s; LDS buffer 1 = slice s+1; R = slice s+2 in flight
      mma(F0, acc);
      rfrag(F1, 1);
      sstore(R, 0);
      gload(R, s + 3);
      schedule();
      __syncthreads();
      // F1 = slice s+1; LDS buffer 0 = slice s+2; R = slice s+3 in flight
      mma(F1, acc);
      rfrag(F0, 0);
      sstore(R, 1);
      gload(R, s + 4);
      schedule();
      __syncthreads();
    }
    if (s < ns) mma(F0, acc);  // odd slice count
  }
};

// Weights in the packed layout (see pack_kernel): each wave loads its own
// weight fragments straight into registers with coalesced 1 KB loads, two
// slices ahead; only the activations (shared by the 4 waves) go through LDS.
// Activations move in pairs of slices: one load instruction covers 8 rows x
// 128 bytes (a whole cache line per row, where a single slice would use half
// of each line and leave the other half to be fetched again), staged in
// registers two slices ahead and stored into one of two LDS pair buffers.
// Every slice is 8*NBW fenced steps, one MFMA each, fenced so the compiler
// keeps this order: MFMA i covers weight band nb = i%NBW, then row block
// mi = (i/NBW)%4, then k half kk = i/(4*NBW) (an accumulator is reused
// 4*NBW MFMAs later; consecutive MFMAs share the activation fragment).
//   after the last MFMA of an activation fragment: read the next slice's
//                fragment into the same registers (one fragment set)
//   after the last MFMA of a weight fragment (row block 3): reload it with
//                slice s+2's
//   even slices only, step kAst: store the staged pair p+1 into LDS;
//                step kAst+2: load pair p+2 into that staging set
template <bool UP, int NBW>
struct PipePacked {
  static constexpr int kSteps = 8 * NBW;
  // 20 (NBW 4); 8 (NBW 2: swept over 2..12 on the 16B shape, up projection
  // 376-377 us at 8 and 10 against 378-381 us at 2, 4, 6 and 12)
  static constexpr int kAst = NBW == 2 ? 8 : kSteps - 12;
  static constexpr int kPairElems = 2 * BM * LDK;                // one pair buffer
  const GemmSeg& g;
  const uint16_t* bb[NBW];
  uint32_t bo[NBW];
  uint32_t arow[4];   // byte offset of this lane's 4 activation rows
  int ns, lane, wave;
  uint16_t* sA;       // 2 pair buffers x 2 slices x BM x LDK

  __device__ __forceinline__ int clampk(int s) const { return s < ns ? s : ns - 1; }
  // Lane l of load i: row 32*wave + 8*i + l/8, 16-byte piece l%8 of the pair
  // (slice 2p + piece/4, piece%4 within it).
  __device__ __forceinline__ void aload(u32x4 (&r)[4], int p) const {
    const int pc = lane & 7;
    const uint32_t o = (uint32_t)clampk(2 * p + (pc >> 2)) * (BK * 2) + (pc & 3) * 16;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = ld_off<u32x4>(g.A, arow[i] + o);
  }
  __device__ __forceinline__ void astore(const u32x4 (&r)[4], int p) const {
    const int pc = lane & 7;
    uint16_t* base = sA + (p & 1) * kPairElems + (pc >> 2) * (BM * LDK) + (pc & 3) * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4*>(&base[(32 * wave + 8 * i + (lane >> 3)) * LDK]) = r[i];
  }
  __device__ __forceinline__ void bload(bf16x8 (&b)[2][NBW], int kk, int nb, int s) const {
    const uint32_t kb = (uint32_t)clampk(s) * 2 + kk;  // 16-wide k block
    b[kk][nb] = ld_off<bf16x8>(bb[nb], bo[nb] + kb * 1024u);
  }
  // fragment of slice s (pair s/2, half s%2)
  __device__ __forceinline__ void rfrag(bf16x8 (&a)[2][4], int kk, int mi, int s) const {
    const int ko = kk * 16 + (lane >> 5) * 8;
    const uint16_t* buf = sA + ((s >> 1) & 1) * kPairElems + (s & 1) * (BM * LDK);
    a[kk][mi] = *reinterpret_cast<const bf16x8*>(&buf[(mi * 32 + (lane & 31)) * LDK + ko]);
  }
  template <bool EVEN>
  __device__ __forceinline__ void slice(int s, bf16x8 (&a)[2][4], bf16x8 (&bc)[2][NBW],
                                        u32x4 (&rs)[4], f32x16 (&acc)[4][NBW]) const {
#pragma unroll
    for (int i = 0; i < kSteps; ++i) {
      const int q = i / NBW, nb = i % NBW, kk = q >> 2, mi = q & 3;
      acc[mi][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bc[kk][nb], a[kk][mi], acc[mi][nb],
                                                            0, 0, 0);
      if (nb == NBW - 1) rfrag(a, kk, mi, s + 1);
      if (mi == 3) bload(bc, kk, nb, s + 2);
      if (EVEN && i == kAst) astore(rs, (s >> 1) + 1);
      if (EVEN && i == kAst + 2) aload(rs, (s >> 1) + 2);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // Loads of one slice's weights (and, for an even slice, of the activation
  // pair two ahead), in the order a steady-state slice issues them.  SKIP0:
  // the first k half's weights are already in flight (first_weights).
  template <bool EVEN, bool SKIP0 = false>
  __device__ __forceinline__ void preload(bf16x8 (&b)[2][NBW], int sb, u32x4 (&r)[4],
                                          int pa) const {
#pragma unroll
    for (int i = 0; i < kSteps; ++i) {
      const int q = i / NBW, nb = i % NBW, kk = q >> 2, mi = q & 3;
      if (mi == 3 && !(SKIP0 && kk == 0)) bload(b, kk, nb, sb);
      if (EVEN && i == kAst + 2) aload(r, pa);
    }
  }
  // Slice 0's first k half of weights: they depend only on the tile's
  // expert and column tile, so they are requested before the activation
  // rows' gather indices are read.
  __device__ __forceinline__ void first_weights(bf16x8 (&b)[2][NBW]) const {
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) bload(b, 0, nb, 0);
  }
  // B0: slice 0's weights with the first k half in flight (first_weights).
  __device__ __forceinline__ void run(f32x16 (&acc)[4][NBW], bf16x8 (&B0)[2][NBW]) const {
    u32x4 R[4];
    bf16x8 A[2][4], B1[2][NBW];
    aload(R, 0);
    astore(R, 0);
    __builtin_amdgcn_sched_barrier(0);
    preload<true, true>(B0, 0, R, 1);
    preload<false>(B1, 1, R, 0);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) rfrag(A, kk, mi, 0);
    int s = 0;
    for (; s + 2 <= ns; s += 2) {
      slice<true>(s, A, B0, R, acc);
      __syncthreads();
      slice<false>(s + 1, A, B1, R, acc);
      __syncthreads();
    }
    if (s < ns) {  // odd slice count: MFMAs only
#pragma unroll
      for (int i = 0; i < kSteps; ++i) {
        const int q = i / NBW, nb = i % NBW, kk = q >> 2, mi = q & 3;
        acc[mi][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(B0[kk][nb], A[kk][mi],
                                                              acc[mi][nb], 0, 0, 0);
      }
    }
  }
};

template <bool UP, bool PACKED, int NBW>
__global__ __launch_bounds__(kThreads, NBW == 2 ? 2 : 1) void gemm_bf16_kernel(GemmArgs args) {
  using TL = Tile<NBW>;
  constexpr int OC = UP ? TL::UPC : TL::BN;  // output columns of the tile
  constexpr int kStage = 64 * (OC + 4);      // epilogue staging tile (elements)
  constexpr int kSB = PACKED ? kStage : (2 * BN * LDK > kStage ? 2 * BN * LDK : kStage);
  // packed weights: two pair buffers (4 slices); row-major: two slices
  __shared__ __attribute__((aligned(16))) uint16_t sA[PACKED ? 4 : 2][BM * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t sB[kSB];

  // Packed weights: the first tile of each group (only segment 0 carries a
  // tile list), read in one batch next to the tile count: lane l holds
  // entries l, l + 64, ... (n_groups + 1 <= 257 of them), so finding a
  // tile's group below takes ballots instead of a chain of dependent loads.
  // (The row-major pipeline has no registers to spare for it and searches.)
  const int lane_id = threadIdx.x & 63;
  int toff[5] = {0, 0, 0, 0, 0};
  if (PACKED && args.seg[0].tile_off) {
    const GemmSeg& gl = args.seg[0];
#pragma unroll
    for (int j = 0; j < 5; ++j) {  // lanes past the end repeat the last entry
      const int i = 64 * j + lane_id;
      toff[j] = gl.tile_off[i < gl.n_groups ? i : gl.n_groups];
    }
  }
  const int G0 = seg_m_tiles(args.seg[0]) * args.seg[0].nN;
  const int G1 = args.nseg > 1 ? seg_m_tiles(args.seg[1]) * args.seg[1].nN : 0;
  const int G = G0 + G1;
  int w = (int)blockIdx.x;
  if (args.steal) {
    w = claim_tile(w, G, G1, args.steal);
    if (w < 0) return;
  } else if (w >= G) {
    return;
  }
  int si, L;
  xcd_remap2(w, G0, G1, si, L);
  const GemmSeg& g = args.seg[si];

  // Logical order within a segment: group, then column tile, then M-tile,
  // so the M-tiles that share a weight tile run next to each other on one XCD.
  int e, nt, row0, rows, mt_deferred = -1;
  if (!PACKED && g.tile_off) {
    int lo = 0, hi = g.n_groups;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (g.tile_off[mid] * g.nN <= L)
        lo = mid;
      else
        hi = mid;
    }
    e = lo;
    const int t0 = g.tile_off[e], te = g.tile_off[e + 1] - t0;
    const int local = L - t0 * g.nN;
    nt = local / te;
    const int mt = t0 + (local - nt * te);
    row0 = g.tile_row0[mt];
    rows = g.tile_rows[mt];
  } else if (g.tile_off) {
    // The group of logical tile L is the last one whose first tile * nN is
    // <= L: the count of such groups, less one (the entries do not
    // decrease).
    const int t0v = toff[0], t1v = toff[1], t2v = toff[2], t3v = toff[3], t4v = toff[4];
    const int nN = g.nN, ng = g.n_groups;
    const int cnt = __popcll(__ballot((lane_id < ng) & (t0v * nN <= L))) +
                    __popcll(__ballot((64 + lane_id < ng) & (t1v * nN <= L))) +
                    __popcll(__ballot((128 + lane_id < ng) & (t2v * nN <= L))) +
                    __popcll(__ballot((192 + lane_id < ng) & (t3v * nN <= L))) +
                    __popcll(__ballot((256 + lane_id < ng) & (t4v * nN <= L)));
    e = cnt - 1;
    auto entry = [&](int i) {  // tile_off[i], i uniform: lane i % 64 of slot i / 64
      const int l = i & 63, j = i >> 6;
      const int r0 = __builtin_amdgcn_readlane(t0v, l), r1 = __builtin_amdgcn_readlane(t1v, l),
                r2 = __builtin_amdgcn_readlane(t2v, l), r3 = __builtin_amdgcn_readlane(t3v, l),
                r4 = __builtin_amdgcn_readlane(t4v, l);
      return j == 0 ? r0 : j == 1 ? r1 : j == 2 ? r2 : j == 3 ? r3 : r4;
    };
    const int t0 = entry(e), te = entry(e + 1) - t0;
    const int local = L - t0 * g.nN;
    nt = local / te;
    mt_deferred = t0 + (local - nt * te);  // its rows are read after the first weights
    row0 = 0;
    rows = 0;
  } else {
    const int num_m = seg_m_tiles(g);
    e = 0;
    nt = L / num_m;
    const int mt = L - nt * num_m;
    row0 = mt * BM;
    rows = (int)(g.single_rows - row0 < BM ? g.single_rows - row0 : BM);
  }

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Activation row r of the tile as a 32-bit byte offset from the uniform
  // base (the ABI keeps every operand below 2^31 elements); rows past the
  // tile's end repeat its last row.
  auto arow_off = [&](int r) -> uint32_t {
    const int rr = r < rows ? r : rows - 1;
    const int64_t grow = (int64_t)row0 + rr;
    const int64_t src = g.a_rows ? (int64_t)g.a_rows[grow] : grow;
    return (uint32_t)(src * g.lda) * 2u;
  };
  const uint16_t* b0base = g.B0 + (int64_t)e * g.b_stride;
  const uint16_t* b1base = UP ? g.B1 + (int64_t)e * g.b_stride : b0base;
  // This wave's weight rows inside the tile: up = UPC/4 W1 rows (and the
  // same W3 rows), down = WN W2 rows.
  const int nr = UP ? wave * (TL::UPC / 4) : wave * TL::WN;

  f32x16 acc[4][NBW];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[mi][nb][j] = 0.f;

  const int ns = g.K / BK;  // K is a multiple of 32
  if constexpr (PACKED) {
    // Packed weights: 32-row bands of 16-wide k blocks (512 elements each).
    const uint32_t KB = (uint32_t)(g.K / 16);
    PipePacked<UP, NBW> pipe{g, {}, {}, {}, ns, lane, wave, &sA[0][0]};
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      // up: bands 0..NBW/2-1 of W1, then the same bands of W3; down: W2
      int brow = UP ? nt * TL::UPC + nr + (nb % (NBW / 2)) * 32 : nt * TL::BN + nr + nb * 32;
      if (brow > g.N - 32) brow = g.N - 32;  // clamped bands: outputs not stored
      pipe.bb[nb] = (UP && nb >= NBW / 2) ? b1base : b0base;
      pipe.bo[nb] = ((uint32_t)(brow >> 5) * KB * 512u + lane * 8) * 2u;
    }
    bf16x8 B0[2][NBW];
    pipe.first_weights(B0);
    __builtin_amdgcn_sched_barrier(0);
    if (mt_deferred >= 0) {
      row0 = g.tile_row0[mt_deferred];
      rows = g.tile_rows[mt_deferred];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) pipe.arow[i] = arow_off(32 * wave + 8 * i + (lane >> 3));
    pipe.run(acc, B0);
  } else {
    static_assert(NBW == 4, "row-major weights take the 128 x 512 tile");
    const int lc = tid & 3, lr = tid >> 2;  // 16-byte chunk of a 32-wide row; row 0..63
    uint32_t aoff[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) aoff[i] = arow_off(lr + 64 * i) + lc * 16u;
    uint32_t boff[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = lr + 64 * i;  // tile row 0..511
      int brow = UP ? nt * kUpCols + (r & (kUpCols - 1)) : nt * BN + r;
      if (brow > g.N - 1) brow = g.N - 1;  // clamped rows: outputs not stored
      boff[i] = ((uint32_t)brow * (uint32_t)g.K + lc * 8) * 2u;
    }
    PipeLds<UP, 4> pipe{g, b0base, b1base, {aoff[0], aoff[1]},
                        {boff[0], boff[1], boff[2], boff[3], boff[4], boff[5], boff[6], boff[7]},
                        ns, nr, lane, lc, lr, sA,
                        reinterpret_cast<uint16_t(*)[BN * LDK]>(&sB[0])};
    pipe.run(acc);
  }

  // 32-row blocks holding at least one real row (uniform over the block).
  // The main loop always computes all four: a second loop specialisation
  // for shorter tiles would not fit the register budget next to this one.
  const int mblocks = (rows + 31) >> 5;

  // Epilogue in two passes of 64 rows through an LDS staging tile (in sB).
  // The MFMAs computed the transposed tile (weights as the first operand),
  // so lane l holds token l % 32 of each 32-row block and, per group of four
  // accumulator registers, four consecutive output columns: one 8-byte LDS
  // write per group.  The staging row pitch (in 4-byte words) is 2 mod 64,
  // so the 32 tokens of a write land in distinct bank pairs.
  constexpr int LDO = OC + 4;
  constexpr int CPR = OC / 8;            // 16-byte chunks per row
  uint16_t* stile = &sB[0];
  const int cbase = nt * OC;
  // what = 0: the output (SwiGLU for the up projection); with g.P (up only),
  // what = 1, 2 also keep the pre-activations W1 x and W3 x for a backward
  // pass, at columns cbase and N + cbase of P.
  const int nwhat = (UP && g.P) ? 3 : 1;
  for (int what = 0; what < nwhat; ++what) {
    uint16_t* dst = what == 0 ? g.C : g.P;
    const int64_t ldd = what == 0 ? g.ldc : 2 * (int64_t)g.N;
    const int coff = cbase + (what == 2 ? g.N : 0);
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      __syncthreads();
#pragma unroll
      for (int mh = 0; mh < 2; ++mh) {
        const int mi = pass * 2 + mh;
        if (mi >= mblocks) continue;
        const int tl = mh * 32 + (lane & 31);
#pragma unroll
        for (int nb = 0; nb < (UP ? NBW / 2 : NBW); ++nb) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int col = nr + nb * 32 + 8 * q + 4 * (lane >> 5);
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float x = acc[mi][nb][4 * q + e];
              if (UP) {
                const float y = acc[mi][nb + NBW / 2][4 * q + e];
                if (what == 0)
                  v[e] = x * __builtin_amdgcn_rcpf(1.0f + __expf(-x)) * y;
                else
                  v[e] = what == 1 ? x : y;
              } else {
                v[e] = x;
              }
            }
            bf16x4 pk = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
            *reinterpret_cast<bf16x4*>(&stile[tl * LDO + col]) = pk;
          }
        }
      }
      __syncthreads();
      for (int c = tid; c < 64 * CPR; c += kThreads) {
        const int rl = c / CPR, ch = c - rl * CPR;
        const int r = pass * 64 + rl;
        if (r < rows && cbase + ch * 8 < g.N) {
          const uint2 lo = *reinterpret_cast<const uint2*>(&stile[rl * LDO + ch * 8]);
          const uint2 hi = *reinterpret_cast<const uint2*>(&stile[rl * LDO + ch * 8 + 4]);
          *reinterpret_cast<u32x4*>(dst + ((int64_t)row0 + r) * ldd + coff + ch * 8) =
              u32x4{lo.x, lo.y, hi.x, hi.y};
        }
      }
    }
  }
}

// fp32 storage: one thread per output element, plain dot products.
struct GemmF32Args {
  const float* A;
  const int32_t* a_rows;
  int64_t lda;
  const float* B0;
  const float* B1;
  int64_t b_stride;
  int K, N;
  float* C;
  int64_t ldc;
  int64_t rows;
  const int32_t* offsets;  // nullable: single group
  int n_groups;
};

template <bool UP>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmF32Args g) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= g.rows * g.N) return;
  const int64_t r = idx / g.N;
  const int c = (int)(idx - r * g.N);
  int e = 0;
  if (g.offsets) {
    int lo = 0, hi = g.n_groups;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (g.offsets[mid] <= r)
        lo = mid;
      else
        hi = mid;
    }
    e = lo;
  }
  const int64_t src = g.a_rows ? (int64_t)g.a_rows[r] : r;
  const float* a = g.A + src * g.lda;
  if (UP) {
    const float* w1 = g.B0 + (int64_t)e * g.b_stride + (int64_t)c * g.K;
    const float* w3 = g.B1 + (int64_t)e * g.b_stride + (int64_t)c * g.K;
    float x1 = 0.f, x3 = 0.f;
    for (int j = 0; j < g.K; ++j) {
      x1 = fmaf(a[j], w1[j], x1);
      x3 = fmaf(a[j], w3[j], x3);
    }
    g.C[r * g.ldc + c] = silu(x1) * x3;
  } else {
    const float* w2 = g.B0 + (int64_t)e * g.b_stride + (int64_t)c * g.K;
    float acc = 0.f;
    for (int j = 0; j < g.K; ++j) acc = fmaf(a[j], w2[j], acc);
    g.C[r * g.ldc + c] = acc;
  }
}

}  // namespace

template <int NBW>
static GemmSeg up_seg(const FfnArgs& a) {
  GemmSeg up{};
  up.A = (const uint16_t*)a.x;
  up.a_rows = a.x_rows;
  up.lda = a.ldx;
  up.B0 = (const uint16_t*)a.w1;
  up.B1 = (const uint16_t*)a.w3;
  up.b_stride = (int64_t)a.d_ff_g * a.d;
  up.K = a.d;
  up.N = a.d_ff_g;
  up.C = (uint16_t*)a.hbuf;
  up.ldc = a.d_ff_g;
  up.P = (uint16_t*)a.preact;
  up.nN = (a.d_ff_g + Tile<NBW>::UPC - 1) / Tile<NBW>::UPC;
  if (a.tiles) {
    up.tile_row0 = a.tiles->row0;
    up.tile_rows = a.tiles->rows;
    up.tile_off = a.tiles->off;
    up.num_tiles = a.tiles->count;
  }
  up.n_groups = a.n_groups;
  up.single_rows = a.rows;
  return up;
}

template <int NBW>
static GemmSeg down_seg(const FfnArgs& a) {
  GemmSeg dn = up_seg<NBW>(a);
  dn.A = (const uint16_t*)a.hbuf;
  dn.a_rows = nullptr;
  dn.lda = a.d_ff_g;
  dn.B0 = (const uint16_t*)a.w2;
  dn.B1 = nullptr;
  dn.b_stride = (int64_t)a.d * a.d_ff_g;
  dn.K = a.d_ff_g;
  dn.N = a.d;
  dn.C = (uint16_t*)a.y;
  dn.ldc = a.d;
  dn.nN = (a.d + Tile<NBW>::BN - 1) / Tile<NBW>::BN;
  return dn;
}

static int max_m_tiles(const FfnArgs& a) {
  return a.tiles ? a.tiles->max_tiles : (int)((a.rows + BM - 1) / BM);
}

template <bool UP, bool PACKED, int NBW>
static hipError_t launch_bf16_t(const FfnArgs* segs, int nseg, hipStream_t s) {
  GemmArgs args{};
  int grid = 0;
  args.nseg = 0;
  for (int i = 0; i < nseg; ++i) {
    if (segs[i].rows == 0) continue;
    // the kernel reads a tile list of segment 0 only
    if (segs[i].tiles && args.nseg > 0) return hipErrorInvalidValue;
    args.seg[args.nseg] = UP ? up_seg<NBW>(segs[i]) : down_seg<NBW>(segs[i]);
    grid += max_m_tiles(segs[i]) * args.seg[args.nseg].nN;
    ++args.nseg;
  }
  if (args.nseg == 0) return hipSuccess;
  // claim counters: with a device tile list that carries them
  const TileList* tl = segs[0].rows > 0 ? segs[0].tiles : nullptr;
  args.steal = tl && tl->steal ? tl->steal + (UP ? 0 : 8) : nullptr;
  hipLaunchKernelGGL((gemm_bf16_kernel<UP, PACKED, NBW>), dim3((unsigned)grid), dim3(kThreads), 0,
                     s, args);
  return hipGetLastError();
}

// Packed weights: both projections take the 128 x 256 tile (d_ff = 1408 is
// 11 of its column tiles, and two workgroups share a CU, so one's prologue
// and epilogue overlap the other's MFMAs and the launch tail is half a tile
// deep).  Row-major weights: 128 x 512 for both.
template <bool UP>
static hipError_t launch_bf16(const FfnArgs* segs, int nseg, bool packed, hipStream_t s) {
  if (!packed) return launch_bf16_t<UP, false, 4>(segs, nseg, s);
  return launch_bf16_t<UP, true, 2>(segs, nseg, s);
}

static hipError_t launch_f32(const FfnArgs& a, bool up, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  if (up) {
    GemmF32Args g{(const float*)a.x, a.x_rows, a.ldx, (const float*)a.w1, (const float*)a.w3,
                  (int64_t)a.d_ff_g * a.d, a.d, a.d_ff_g, (float*)a.hbuf, a.d_ff_g, a.rows,
                  a.tiles ? a.offsets : nullptr, a.n_groups};
    const int64_t n = a.rows * a.d_ff_g;
    hipLaunchKernelGGL(gemm_f32_kernel<true>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       s, g);
  } else {
    GemmF32Args g{(const float*)a.hbuf, nullptr, a.d_ff_g, (const float*)a.w2, nullptr,
                  (int64_t)a.d * a.d_ff_g, a.d_ff_g, a.d, (float*)a.y, a.d, a.rows,
                  a.tiles ? a.offsets : nullptr, a.n_groups};
    const int64_t n = a.rows * a.d;
    hipLaunchKernelGGL(gemm_f32_kernel<false>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       s, g);
  }
  return hipGetLastError();
}

hipError_t launch_ffn_up(const FfnArgs* segs, int nseg, hipStream_t s) {
  if (segs[0].dtype == 0) {
    for (int i = 0; i < nseg; ++i) {
      const hipError_t e = launch_f32(segs[i], true, s);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  return launch_bf16<true>(segs, nseg, segs[0].packed, s);
}

hipError_t launch_ffn_down(const FfnArgs* segs, int nseg, hipStream_t s) {
  if (segs[0].dtype == 0) {
    for (int i = 0; i < nseg; ++i) {
      const hipError_t e = launch_f32(segs[i], false, s);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  return launch_bf16<false>(segs, nseg, segs[0].packed, s);
}

hipError_t launch_pack(const void* src, void* dst, int64_t rows, int K, hipStream_t s) {
  const int64_t n = rows * (K / 8);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     (const uint16_t*)src, (uint16_t*)dst, rows, K);
  return hipGetLastError();
}

hipError_t launch_grouped_ffn(const FfnArgs& a, hipStream_t s) {
  const hipError_t e = launch_ffn_up(&a, 1, s);
  if (e != hipSuccess) return e;
  return launch_ffn_down(&a, 1, s);
}

}  // namespace moe
