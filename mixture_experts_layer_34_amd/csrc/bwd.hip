// Backward pass of the MoE layer on gfx950.
//
// The products of the backward (the chain rule of SwiGLU experts, the
// gate-weighted combine, the softmax router and the expert-level balance
// loss) go through two MFMA kernels.  bg_kernel: rows grouped by expert,
// 128 x 128 output tiles, 64-deep K slices staged through LDS with the next
// slices' global loads in flight, four waves of 64 x 64 each (2 x 2 blocks
// of 32x32x16 bf16 MFMAs, fp32 accumulators).  wgrad_kernel: the weight
// gradients, each expert reducing over its own rows, on 256 x 128 tiles.
// Operands that are K-strided in memory (weights read against their stored
// orientation, activations reduced over tokens) are transposed on their way
// into LDS; see lpos() for the bank layout.
#include "bwd.h"
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int BM = kBgTile, BN = kBgTile, BK = kBgK;
// One staged operand tile (BM rows of BK elements, see lpos), with room for
// the epilogue's fp32 staging (four waves x 32 rows x 68 floats over the two
// buffers of sA).
constexpr int kStageF32El = 4 * 32 * (64 + 4) * 2;
constexpr int TILE_EL = BM * BK > kStageF32El / 2 ? BM * BK : kStageF32El / 2;
constexpr int NT = 256;

enum { EPI_F32 = 0, EPI_BF16 = 1, EPI_SWIGLU = 2, EPI_DU = 3 };

// LDS layout of a staged tile: row m holds its 64 K elements as eight
// 16-byte chunks at 128-byte pitch, chunk c at position c ^ swz(m).  Measured
// on gfx950 (bank-conflict counters on single access patterns): a 16-byte
// read is served in four passes of 16 lanes (lane bit 5, and the parity of
// lane bits 2..4) over 64 four-byte banks, and an 8-byte write in passes of
// 16 consecutive lanes over 32 banks.  The MFMA fragment reads (lane l on
// row l % 32) then need swz to take 8 values on the even rows of each pass,
// and the transposing stores (4 rows 8 apart, or 2 rows 8 apart, per pass)
// need rows differing in bits 3 and 4 on disjoint chunks; this swz does both
// (4 cycles per read and per 8-byte write, against 8 for the padded pitch it
// replaces).
__device__ __forceinline__ int swz(int m) {
  return ((m >> 1) & 1) | (((m >> 4) & 1) << 1) | (((m >> 3) & 1) << 2);
}
__device__ __forceinline__ int lpos(int m, int c) { return m * BK + ((c ^ swz(m)) << 3); }

struct BgArgs {
  BgSeg seg[kBgMaxSeg];
  int bound[kBgMaxSeg];  // tiles of each segment (an upper bound for a tile list)
  int nseg;
};

// Workgroup -> (segment, logical tile).  Workgroups are dealt round-robin
// over the 8 XCDs; each XCD takes an even share of every segment's tiles, in
// segment order, as one contiguous range of logical tiles (grouped by expert,
// then column tile), so the tiles that share activation rows and weight
// tiles run on one XCD and meet in its L2.  Returns false for workgroups
// beyond the live tiles.
__device__ __forceinline__ bool xcd_pick(const BgArgs& a, int tile, int& si, int& L) {
  constexpr int kXcd = 8;
  const int bid = (int)blockIdx.x, x = bid % kXcd;
  int i = bid / kXcd;
  for (int s = 0; s < a.nseg; ++s) {
    const BgSeg& g = a.seg[s];
    const int G = g.t_off ? *g.t_count * ((g.N + tile - 1) / tile) : a.bound[s];
    const int q = G / kXcd, r = G % kXcd;
    const int share = q + (x < r ? 1 : 0);
    if (i < share) {
      si = s;
      L = x * q + (x < r ? x : r) + i;
      return true;
    }
    i -= share;
  }
  return false;
}

// ---- K-contiguous operand: the tile's 128 rows x 64 k.  Thread chunk
// tid + 256 i covers row (tid >> 3) + 32 i and k (tid & 7) * 8 .. + 7.
struct KcRows {
  uint32_t off[4];  // byte offset of the row's first element
  uint32_t ok;      // bit i: row i exists
};

// Packed weights (moe_pack_weights): a [rows][K] matrix stored as 32-row
// bands of 16-wide K blocks of 512 elements, element (r, k) of a block at
// ((r % 32) + 32 ((k % 16) / 8)) * 8 + k % 8.  Eight consecutive k of one
// row stay contiguous, which is all the loaders below read.
__device__ __forceinline__ int64_t packed_at(int64_t r, int k, int64_t K) {
  return ((r >> 5) * (K >> 4) + (k >> 4)) * 512 + ((r & 31) + 32 * ((k >> 3) & 1)) * 8 + (k & 7);
}

// PK: the operand is a packed weight matrix (K-contiguous in the packed
// sense); a 64-wide K slice then moves the 16-byte pieces by 64 * 32
// elements instead of 64.
template <bool PK = false>
__device__ __forceinline__ void kc_init(KcRows& R, int tid, int nvalid, int64_t row0,
                                        int64_t ld) {
  R.ok = 0;
  const int kc = (tid & 7) * 8;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (tid >> 3) + 32 * i;
    const bool v = r < nvalid;
    const int64_t mr = v ? row0 + r : 0;
    R.off[i] = (uint32_t)((PK ? packed_at(mr, kc, ld) : mr * ld + kc) * 2);
    R.ok |= (v ? 1u : 0u) << i;
  }
}

template <bool PK = false>
__device__ __forceinline__ void kc_load(u32x4 v[4], const void* base, const KcRows& R, int k0,
                                        int klim, int tid) {
  const bool kin = k0 + (tid & 7) * 8 < klim;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (kin && ((R.ok >> i) & 1u))
      v[i] = ld_off<u32x4>(base, R.off[i] + (uint32_t)k0 * (PK ? 64u : 2u));
    else
      v[i] = u32x4{0u, 0u, 0u, 0u};
  }
}

__device__ __forceinline__ void kc_store(uint16_t* s, const u32x4 v[4], int tid) {
  const int kc = (tid & 7) * 8;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (tid >> 3) + 32 * i;
    *reinterpret_cast<u32x4*>(&s[lpos(r, kc >> 3)]) = v[i];
  }
}

// ---- K-strided operand: 64 k rows x 128 columns of the tile.  Thread:
// columns mb*8 .. +7, k rows kg*4 .. +3.  Row-major: mb = 4 wave + lane % 4,
// kg = lane / 4, so four lanes read 64 contiguous bytes of a row (16 rows per
// load instruction; both other assignments tried, a whole 128-byte row per 8
// lanes and 8 k groups per column block, measured slower).  Packed (32-row
// bands of 16-wide k blocks, 1 KB each, consecutive along k): mb = lane / 8 +
// 8 (wave & 1), kg = lane % 8 + 8 (wave / 2), so a wave's four loads cover
// one band's four consecutive blocks, 4 KB of contiguous memory, instead of
// two 2 KB pieces of two bands (dgrad with packed weights 10 % faster).  The
// transposing LDS stores below stay on distinct banks either way (measured:
// 4 cycles per 8-byte store instruction).  Rows are addressed directly: a row map would put a
// dependent load in front of every load, and the in-order load counter would
// then wait for all loads in flight.
template <bool PK>
__device__ __forceinline__ int ks_mb(int tid) {
  return PK ? ((tid & 63) >> 3) + 8 * ((tid >> 6) & 1) : 4 * (tid >> 6) + (tid & 3);
}
template <bool PK>
__device__ __forceinline__ int ks_kg(int tid) {
  return PK ? (tid & 7) + 8 * (tid >> 7) : (tid & 63) >> 2;
}

template <bool PK = false>
__device__ __forceinline__ void ks_load(u32x4 v[4], const void* base, int64_t ld, int kbase,
                                        int klim, int col0, int clim, int tid) {
  const int mb = ks_mb<PK>(tid), kg = ks_kg<PK>(tid);
  const int col = col0 + mb * 8;
  const bool cin = col < clim;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int kr = kbase + kg * 4 + kk;
    if (cin && kr < klim)
      v[kk] = ld_off<u32x4>(
          base, (uint32_t)((PK ? packed_at(kr, col, ld) : (int64_t)kr * ld + col) * 2));
    else
      v[kk] = u32x4{0u, 0u, 0u, 0u};
  }
}

// Transposes the thread's 4 (k) x 8 (columns) block into LDS rows = columns
// (rows roff + 0 .. 127 of the staged tile); PK as in the ks_load that
// filled v.
template <bool PK = false>
__device__ __forceinline__ void ks_store(uint16_t* s, const u32x4 v[4], int tid, int roff = 0) {
  const int mb = ks_mb<PK>(tid), kg = ks_kg<PK>(tid);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int w = i >> 1, sh = (i & 1) * 16;
    const uint32_t lo = ((v[0][w] >> sh) & 0xFFFFu) | (((v[1][w] >> sh) & 0xFFFFu) << 16);
    const uint32_t hi = ((v[2][w] >> sh) & 0xFFFFu) | (((v[3][w] >> sh) & 0xFFFFu) << 16);
    *reinterpret_cast<uint2*>(&s[lpos(roff + mb * 8 + i, kg >> 1) + (kg & 1) * 4]) =
        make_uint2(lo, hi);
  }
}

__device__ __forceinline__ uint2 pack4(float a, float b, float c, float d) {
  return make_uint2((uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16),
                    (uint32_t)f32_to_bf16(c) | ((uint32_t)f32_to_bf16(d) << 16));
}

__device__ __forceinline__ void unpack4(uint2 p, float* o) {
  o[0] = bf16_to_f32((uint16_t)(p.x & 0xFFFFu));
  o[1] = bf16_to_f32((uint16_t)(p.x >> 16));
  o[2] = bf16_to_f32((uint16_t)(p.y & 0xFFFFu));
  o[3] = bf16_to_f32((uint16_t)(p.y >> 16));
}

// Rows grouping (the tile list of the forward's grouping, or one group of
// `rows` rows).  A is K-contiguous; BKS: B K-strided in memory; DUAL: second
// B with its own accumulators (SwiGLU's a and b); PK: B (and B2) packed.
// SB: one staged slice and one register set, so the dual product (128
// accumulators) fits two workgroups per CU instead of one and the single
// product three instead of two; the other workgroups' MFMAs then run while
// one stages a slice (16B: a/b recompute 776 -> 570 us, q 305 -> 272 us,
// dx 540-560 -> 513-523 us).
template <bool BKS, int EPI, bool DUAL, bool PK, bool SB = false>
__global__ __launch_bounds__(NT, DUAL ? (SB ? 2 : 1) : (SB ? 3 : 2)) void bg_kernel(BgArgs args) {
  static_assert(!SB || EPI == EPI_SWIGLU || EPI == EPI_BF16,
                "single-buffered tiles stage at most the bf16 epilogue");
  constexpr int NBUF = SB ? 1 : 2;
  // a single sA buffer also holds the bf16 epilogue's staging (4 x 32 x 72)
  constexpr int TEA = (SB && TILE_EL < 4 * 32 * 72) ? 4 * 32 * 72 : TILE_EL;
  __shared__ __attribute__((aligned(16))) uint16_t sA[NBUF][TEA];
  __shared__ __attribute__((aligned(16))) uint16_t sB[NBUF][TILE_EL];
  __shared__ __attribute__((aligned(16))) uint16_t sB2[DUAL ? NBUF : 1][DUAL ? TILE_EL : 8];

  int si = 0, L = 0;
  if (!xcd_pick(args, BN, si, L)) return;
  const BgSeg& g = args.seg[si];
  const int nN = (g.N + BN - 1) / BN;

  int e = 0, nt, mt, m0, mvalid;
  if (g.t_off) {
    int lo = 0, hi = g.n_groups;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (g.t_off[mid] * nN <= L)
        lo = mid;
      else
        hi = mid;
    }
    e = lo;
    const int t0 = g.t_off[e], te = g.t_off[e + 1] - t0;
    const int local = L - t0 * nN;
    nt = local / te;
    mt = t0 + (local - nt * te);
    m0 = g.t_row0[mt];
    mvalid = g.t_rows[mt];
  } else {
    const int num_m = (int)((g.rows + BM - 1) / BM);
    nt = L / num_m;
    mt = L - nt * num_m;
    m0 = mt * BM;
    mvalid = (int)(g.rows - m0 < BM ? g.rows - m0 : BM);
  }
  const int kb = 0, ke = g.K;
  const int n0 = nt * BN;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;

  // Row maps of the K-contiguous operands (fixed across K slices).
  KcRows ar{}, br{}, br2{};
  kc_init(ar, tid, mvalid, m0, g.lda);
  if constexpr (!BKS) {
    kc_init<PK>(br, tid, g.N - n0, n0, g.ldb);
    if constexpr (DUAL) br2 = br;
  }
  (void)br2;

  f32x16 acc[2][2], acc2[DUAL ? 2 : 1][DUAL ? 2 : 1];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[nb][mb][j] = 0.0f;
      if constexpr (DUAL) {
#pragma unroll
        for (int j = 0; j < 16; ++j) acc2[nb][mb][j] = 0.0f;
      }
    }

  // Fragment rows of this lane (LDS element offsets of k step 0; step kk
  // is at offset ^ 16 kk).
  int fa[2], fb[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    fa[i] = lpos(wm * 64 + i * 32 + (lane & 31), lane >> 5);
    fb[i] = lpos(wn * 64 + i * 32 + (lane & 31), lane >> 5);
  }

  const int nk = ke > kb ? (ke - kb + BK - 1) / BK : 0;
  // K slices kt+1 and kt+2 wait in registers (two sets, filled in turn)
  // while slice kt is multiplied out of LDS; SB: slice kt+1 in one set.
  constexpr int PF = SB ? 1 : 2;
  for (int p = 0; p < g.npass && nk > 0; ++p) {
    const void* Ab = g.A[p];
    const void* Bb =
        static_cast<const void*>(static_cast<const uint16_t*>(g.B[p]) + (int64_t)e * g.b_gstride);
    const void* B2b = nullptr;
    if constexpr (DUAL)
      B2b = static_cast<const void*>(static_cast<const uint16_t*>(g.B2) +
                                     (int64_t)e * g.b_gstride);
    const int bklim = g.bk_lim;

    u32x4 ra[PF][4], rbv[PF][4], rb2[PF][DUAL ? 4 : 1];
    auto load = [&](int kt, int st) {
      const int k0 = kb + kt * BK;
      kc_load(ra[st], Ab, ar, k0, ke, tid);
      if constexpr (BKS) {
        ks_load<PK>(rbv[st], Bb, g.ldb, k0, bklim, n0, g.b_lim, tid);
        if constexpr (DUAL) ks_load<PK>(rb2[st], B2b, g.ldb, k0, bklim, n0, g.b_lim, tid);
      } else {
        kc_load<PK>(rbv[st], Bb, br, k0, ke, tid);
        if constexpr (DUAL) kc_load<PK>(rb2[st], B2b, br2, k0, ke, tid);
      }
    };
    auto store = [&](int st, int b) {
      kc_store(sA[b], ra[st], tid);
      if constexpr (BKS) {
        ks_store<PK>(sB[b], rbv[st], tid);
        if constexpr (DUAL) ks_store<PK>(sB2[b], rb2[st], tid);
      } else {
        kc_store(sB[b], rbv[st], tid);
        if constexpr (DUAL) kc_store(sB2[b], rb2[st], tid);
      }
    };
    auto compute = [&](int b) {
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        bf16x8 af[2], bfr[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          af[i] = *reinterpret_cast<const bf16x8*>(&sA[b][fa[i] ^ (kk * 16)]);
          bfr[i] = *reinterpret_cast<const bf16x8*>(&sB[b][fb[i] ^ (kk * 16)]);
        }
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
            acc[nb][mb] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[nb], af[mb], acc[nb][mb], 0, 0, 0);
        if constexpr (DUAL) {
          bf16x8 b2[2];
#pragma unroll
          for (int i = 0; i < 2; ++i)
            b2[i] = *reinterpret_cast<const bf16x8*>(&sB2[b][fb[i] ^ (kk * 16)]);
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
              acc2[nb][mb] =
                  __builtin_amdgcn_mfma_f32_32x32x16_bf16(b2[nb], af[mb], acc2[nb][mb], 0, 0, 0);
        }
      }
    };

    // The slice count is padded to even (a padded slice loads zeros) and
    // every step issues its prefetch, clamped to the last slice: a load
    // under a branch leaves the compiler unsure how many loads are in flight
    // where the paths merge, and it then waits for all of them.
    if constexpr (SB) {
      // slice kt + 1 loads while slice kt is multiplied, then takes its
      // place in LDS
      load(0, 0);
      store(0, 0);
      __syncthreads();
      for (int kt = 0; kt < nk; ++kt) {
        load(kt + 1 < nk ? kt + 1 : nk - 1, 0);
        compute(0);
        __syncthreads();
        if (kt + 1 < nk) {
          store(0, 0);
          __syncthreads();
        }
      }
    } else {
      const int nkp = (nk + 1) & ~1;
      load(0, 0);
      load(1 % PF, 1 % PF);
      store(0, 0);
      __syncthreads();
      // Unrolled by two so register sets and LDS buffers are static: slice
      // kt = base + j sits in set j and LDS buffer j.
      for (int base = 0; base < nkp; base += 2) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int kt = base + j;
          load(kt + 2 < nkp ? kt + 2 : nkp - 1, j % PF);
          compute(j % NBUF);
          if (kt + 1 < nkp) store((j ^ 1) % PF, (j ^ 1) % NBUF);
          __syncthreads();
        }
      }
    }
  }

  // Epilogue.  Accumulator element 4q + j of block (nb, mb) is row
  // wm*64 + mb*32 + lane % 32 and column wn*64 + nb*32 + 8q + 4 (lane / 32) + j.
  const int cbase = n0 + wn * 64 + 4 * (lane >> 5);
  (void)cbase;
  // Plain and du epilogues go through LDS, 32 rows of the wave's block at a
  // time: in the accumulator layout each lane holds a different row, so
  // direct accesses would touch 32 rows per instruction; staged, the global
  // loads and stores run along rows.
  constexpr int SPF = 64 + 4;  // fp32 staging pitch (floats)
  constexpr int SPH = 64 + 8;  // bf16 staging pitch (elements)
  static_assert((SB || 4 * 32 * SPF * 2 <= NBUF * TEA) && 4 * 32 * SPH <= NBUF * TEA,
                "epilogue staging fits the buffers of sA");
  if constexpr (EPI == EPI_F32 || EPI == EPI_BF16) {
    char* C = static_cast<char*>(g.C);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      if constexpr (EPI == EPI_F32) {
        float* st = reinterpret_cast<float*>(&sA[0][0]) + wave * 32 * SPF;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x16& a = acc[nb][mb];
            *reinterpret_cast<float4*>(&st[(lane & 31) * SPF + nb * 32 + 8 * q + 4 * (lane >> 5)]) =
                make_float4(a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]);
          }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int r = 4 * i + (lane >> 4), ml = wm * 64 + mb * 32 + r;
          const int c = n0 + wn * 64 + 4 * (lane & 15);
          if (ml < mvalid && c < g.N)
            *reinterpret_cast<float4*>(C + (((int64_t)m0 + ml) * g.ldc + c) * 4) =
                *reinterpret_cast<const float4*>(&st[r * SPF + 4 * (lane & 15)]);
        }
      } else {
        uint16_t* st = &sA[0][0] + wave * 32 * SPH;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x16& a = acc[nb][mb];
            *reinterpret_cast<uint2*>(&st[(lane & 31) * SPH + nb * 32 + 8 * q + 4 * (lane >> 5)]) =
                pack4(a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]);
          }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 8 * i + (lane >> 3), ml = wm * 64 + mb * 32 + r;
          const int c = n0 + wn * 64 + 8 * (lane & 7);
          if (ml < mvalid && c < g.N)
            *reinterpret_cast<u32x4*>(C + (((int64_t)m0 + ml) * g.ldc + c) * 2) =
                *reinterpret_cast<const u32x4*>(&st[r * SPH + 8 * (lane & 7)]);
        }
      }
      __syncthreads();
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    const uint16_t* Q = static_cast<const uint16_t*>(g.q);
    uint16_t* DA = static_cast<uint16_t*>(g.da);
    uint16_t* DB = static_cast<uint16_t*>(g.db);
    uint16_t* GH = static_cast<uint16_t*>(g.gh);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int ml = wm * 64 + mb * 32 + (lane & 31);
      const bool rin = ml < mvalid;
      const int64_t row = (int64_t)m0 + (rin ? ml : 0);
      const float gt = (g.gate && rin) ? g.gate[row] : 1.0f;
      float part = 0.0f;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = cbase + nb * 32 + 8 * q;
          if (!rin || c >= g.N) continue;
          const int64_t at = row * g.ldc + c;
          float qv[4];
          unpack4(*reinterpret_cast<const uint2*>(&Q[at]), qv);
          float da[4], db[4], gh[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float a = acc[nb][mb][4 * q + j], b = acc2[nb][mb][4 * q + j];
            const float sg = 1.0f / (1.0f + __expf(-a));
            const float sl = a * sg;
            const float dsl = sg * (1.0f + a * (1.0f - sg));
            const float hid = sl * b;
            da[j] = gt * qv[j] * b * dsl;
            db[j] = gt * qv[j] * sl;
            gh[j] = gt * hid;
            part += qv[j] * hid;
          }
          *reinterpret_cast<uint2*>(&DA[at]) = pack4(da[0], da[1], da[2], da[3]);
          *reinterpret_cast<uint2*>(&DB[at]) = pack4(db[0], db[1], db[2], db[3]);
          *reinterpret_cast<uint2*>(&GH[at]) = pack4(gh[0], gh[1], gh[2], gh[3]);
        }
      if (g.gate) {
        part += __shfl_xor(part, 32);
        if (rin && lane < 32) g.dgp[row * g.ldgp + nt * 2 + wn] = part;
      }
    }
  } else {  // EPI_DU
    const uint16_t* R = static_cast<const uint16_t*>(g.resid);
    const uint16_t* S = static_cast<const uint16_t*>(g.dxs);
    const uint16_t* X = static_cast<const uint16_t*>(g.dxp);
    float* C = static_cast<float*>(g.C);
    float* st = reinterpret_cast<float*>(&sA[0][0]) + wave * 32 * SPF;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x16& a = acc[nb][mb];
          *reinterpret_cast<float4*>(&st[(lane & 31) * SPF + nb * 32 + 8 * q + 4 * (lane >> 5)]) =
              make_float4(a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]);
        }
      __syncthreads();
      const int c = n0 + wn * 64 + 4 * (lane & 15);
#pragma unroll 2
      for (int i = 0; i < 8; ++i) {
        // The 16 lanes of a row group share the row; for k <= 16 lane j of
        // the group loads slot j's grouped row index and the group trades
        // them by shuffles, so that all k row loads are in flight at once
        // (one dependent index load per slot would serialise them).
        const int r = 4 * i + (lane >> 4), ml = wm * 64 + mb * 32 + r;
        const bool rok = ml < mvalid;
        const int64_t t = (int64_t)m0 + (rok ? ml : 0), at = t * g.ldc + c;
        const bool fast = g.k <= 16;
        const int mys = (fast && rok && (lane & 15) < g.k) ? g.slot_of[t * g.k + (lane & 15)] : -1;
        uint2 xv[16];
        if (fast) {
#pragma unroll
          for (int sl = 0; sl < 16; ++sl) {
            const int rr = __shfl(mys, (lane & 48) | sl);
            xv[sl] = (sl < g.k && rr >= 0 && c < g.N)
                         ? *reinterpret_cast<const uint2*>(&X[(int64_t)rr * g.ldc + c])
                         : make_uint2(0u, 0u);
          }
        }
        if (!rok || c >= g.N) continue;
        const float4 v = *reinterpret_cast<const float4*>(&st[r * SPF + 4 * (lane & 15)]);
        float o[4] = {v.x, v.y, v.z, v.w}, tmp[4];
        if (R) {
          unpack4(*reinterpret_cast<const uint2*>(&R[at]), tmp);
#pragma unroll
          for (int j = 0; j < 4; ++j) o[j] += tmp[j];
        }
        if (S) {
          unpack4(*reinterpret_cast<const uint2*>(&S[at]), tmp);
#pragma unroll
          for (int j = 0; j < 4; ++j) o[j] += tmp[j];
        }
        if (fast) {
          // slots left out by the grouping (index < 0) loaded zeros
#pragma unroll
          for (int sl = 0; sl < 16; ++sl) {
            unpack4(xv[sl], tmp);
#pragma unroll
            for (int j = 0; j < 4; ++j) o[j] += tmp[j];
          }
        } else {
          for (int sl = 0; sl < g.k; ++sl) {
            const int64_t rr = g.slot_of[t * g.k + sl];
            if (rr < 0) continue;  // slot left out by the grouping
            unpack4(*reinterpret_cast<const uint2*>(&X[rr * g.ldc + c]), tmp);
#pragma unroll
            for (int j = 0; j < 4; ++j) o[j] += tmp[j];
          }
        }
        *reinterpret_cast<float4*>(&C[at]) = make_float4(o[0], o[1], o[2], o[3]);
      }
      __syncthreads();
    }
  }
}

// Weight gradients (k grouping, both operands K-strided, fp32 out) on
// 256 x 128 tiles: an expert's K range is only its rows (a few hundred), so
// a tile reuses each staged slice over twice the output of the 128 x 128
// kernel, and each wave's 128 x 64 block (8 accumulator blocks) takes 8
// MFMAs per 6 fragment reads.  Two persistent workgroups per CU (one K
// slice staged at a time, 50 KB of LDS and 252 registers each) taking tiles
// from work queues: one workgroup's slice staging, barriers and epilogue
// run beside the other's MFMAs (measured 10 % faster than one 256 x 256
// workgroup per CU with two staged slices).
//
// Queues: one per XCD (workgroup b runs on XCD b % 8).  XCD x's queue holds
// the experts e = x, x + 8, ... of the segments with a row-offset table
// (all their tiles, expert by expert, so the tiles that read one expert's
// rows meet in one L2) and an eighth of every other segment's tiles, in
// segment order otherwise.  A workgroup whose queue is empty takes tiles
// from the other queues, so tiles of unequal length (each expert reduces
// over its own rows) still balance.
//
// The next tile's first slice is loaded during the current tile's last one,
// before the epilogue's stores: the load counter counts stores too, and a
// wait for a load issued after them would wait for them all.  Expert row
// offsets are read from LDS for the same reason (a global load of them at a
// tile's start would wait for the previous tile's stores).
constexpr int WBM = 256, WBN = 128;  // weight-gradient tile (M x N)
constexpr int WTILE_EL = (WBM + WBN) * BK;  // one staged slice of both operands
constexpr int kWgSP = 64 + 4;                // epilogue staging pitch (floats)
static_assert(4 * 32 * kWgSP * 2 <= WTILE_EL, "four waves' epilogue staging fits the slice");
constexpr int kWgMaxGroups = 256;
constexpr int kXcds = kWgQueues;
// Buffer resource word 3 for raw 32-bit accesses on gfx9, and an offset
// past any output (outputs stay below 2 GiB).
constexpr int kBufWord3 = 0x00020000;
constexpr int kBufDrop = kBwdOutBytes;

struct WTile {
  int si, e, m0, n0, kb, ke, nk;
};

__device__ __forceinline__ int wg_tiles(const BgSeg& g) {
  return ((g.M + WBM - 1) / WBM) * ((g.N + WBN - 1) / WBN);  // per group
}

// Segments [k0, k1) carry the row-offset table (contiguous, same G; k0 = k1
// when none does).
struct WQueues {
  int k0, k1, per_e;  // per_e: tiles of one expert over those segments
};

__device__ __forceinline__ WQueues wqueues(const BgArgs& a) {
  WQueues q{a.nseg, a.nseg, 0};
  bool found = false;
  for (int s = 0; s < a.nseg; ++s)
    if (a.seg[s].koff) {
      if (!found) q.k0 = s;
      found = true;
      q.k1 = s + 1;
      q.per_e += wg_tiles(a.seg[s]);
    }
  return q;
}

// Tiles in XCD x's queue.
__device__ __forceinline__ int wq_count(const BgArgs& a, const WQueues& q, int x) {
  int c = 0;
  for (int s = 0; s < a.nseg; ++s) {
    if (s >= q.k0 && s < q.k1) continue;
    const int S = a.bound[s];
    c += (x + 1) * S / kXcds - x * S / kXcds;
  }
  if (q.k1 > q.k0) {
    const int G = a.seg[q.k0].G;
    c += (G > x ? (G - x + kXcds - 1) / kXcds : 0) * q.per_e;
  }
  return c;
}

// Entry i of XCD x's queue -> segment s and tile t within it (tile t of a
// segment: group t / (nM nN), then column tile, then row tile).
__device__ __forceinline__ void wq_tile(const BgArgs& a, const WQueues& q, int x, int i, int& s,
                                        int& t) {
  for (s = 0; s < a.nseg; ++s) {
    if (s == q.k0 && q.k1 > q.k0) {
      const int G = a.seg[s].G;
      const int ne = G > x ? (G - x + kXcds - 1) / kXcds : 0;
      if (i < ne * q.per_e) {
        const int e = x + kXcds * (i / q.per_e);
        int r = i - (i / q.per_e) * q.per_e;
        while (r >= wg_tiles(a.seg[s])) {
          r -= wg_tiles(a.seg[s]);
          ++s;
        }
        t = e * wg_tiles(a.seg[s]) + r;
        return;
      }
      i -= ne * q.per_e;
      s = q.k1 - 1;
      continue;
    }
    const int S = a.bound[s];
    const int lo = x * S / kXcds, c = (x + 1) * S / kXcds - lo;
    if (i < c) {
      t = lo + i;
      return;
    }
    i -= c;
  }
  s = a.nseg - 1;
  t = 0;  // not reached for i below wq_count
}

// Segment s, tile t -> its coordinates; koff[] holds the one row-offset
// table the launch's segments share.
__device__ __forceinline__ WTile wtile_of(const BgArgs& a, const int* koff, int s, int t) {
  WTile w{};
  const BgSeg& g = a.seg[s];
  const int nN = (g.N + WBN - 1) / WBN, nM = (g.M + WBM - 1) / WBM;
  w.si = s;
  w.e = t / (nM * nN);
  const int r = t - w.e * nM * nN;
  const int nt = r / nM, mt = r - nt * nM;
  w.m0 = mt * WBM;
  w.n0 = nt * WBN;
  if (g.koff) {
    w.kb = koff[w.e];
    w.ke = koff[w.e + 1];
  } else {
    w.kb = w.e * g.kchunk;
    w.ke = w.kb + g.kchunk < g.K ? w.kb + g.kchunk : g.K;
  }
  w.nk = w.ke > w.kb ? (w.ke - w.kb + BK - 1) / BK : 0;
  return w;
}

// A queue entry for s_next: XCD in the top bits, -1 for none.
__device__ __forceinline__ int wq_pack(int x, int i) { return (x << 24) | i; }

__global__ __launch_bounds__(NT, 2) void wgrad_kernel(BgArgs args, int* __restrict__ ctr) {
  // One staged K slice of both operands (A: 256 rows, B: 128 rows); it also
  // holds the epilogue's staging.  Single-buffered, so two workgroups fit a
  // CU and one's LDS staging, barriers and epilogue run beside the other's
  // MFMAs.
  __shared__ __attribute__((aligned(16))) uint16_t sT[WTILE_EL];
  __shared__ int s_koff[kWgMaxGroups + 1];
  __shared__ int s_next[2];
  uint16_t* const sTa = sT;
  uint16_t* const sTb = sT + WBM * BK;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;  // 128 x 64 block of the tile
  int fa[4], fb[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) fa[i] = lpos(wm * 128 + i * 32 + (lane & 31), lane >> 5);
#pragma unroll
  for (int i = 0; i < 2; ++i) fb[i] = lpos(wn * 64 + i * 32 + (lane & 31), lane >> 5);
  const WQueues wq = wqueues(args);
  if (wq.k1 > wq.k0) {
    const int32_t* koff = args.seg[wq.k0].koff;
    for (int i = tid; i <= args.seg[wq.k0].G; i += NT) s_koff[i] = koff[i];
  }
  // Thread 0 alone talks to the queues: it takes from queue qx, and moves to
  // the next nonempty queue when qx runs dry.
  int qx = (int)blockIdx.x % kXcds;
  auto take_sync = [&](int from) -> int {
    for (int k = 0; k < kXcds; ++k) {
      const int x = (from + k) % kXcds;
      const int i = atomicAdd(&ctr[x], 1);
      if (i < wq_count(args, wq, x)) {
        qx = x;
        return wq_pack(x, i);
      }
    }
    return -1;
  };
  u32x4 ra[2][4], rbv[4];
  auto load = [&](const WTile& w, int kt) {
    const BgSeg& g = args.seg[w.si];
    const int k0 = w.kb + kt * BK;
#pragma unroll
    for (int h = 0; h < 2; ++h) ks_load(ra[h], g.A[0], g.lda, k0, w.ke, w.m0 + 128 * h, g.a_lim, tid);
    ks_load(rbv, g.B[0], g.ldb, k0, w.ke, w.n0, g.b_lim, tid);
  };
  auto store = [&]() {
#pragma unroll
    for (int h = 0; h < 2; ++h) ks_store(sTa, ra[h], tid, 128 * h);
    ks_store(sTb, rbv, tid);
  };

  // Tile j of this workgroup finds tile j + 1's entry in s_next[(j + 1) & 1]
  // and fetches tile j + 2's into s_next[j & 1].
  int cur = 0;
  if (tid == 0) {
    cur = take_sync(qx);
    s_next[1] = cur < 0 ? -1 : take_sync(qx);
    s_next[0] = cur;
  }
  __syncthreads();
  cur = s_next[0];
  if (cur < 0) return;  // no tile at all (uniform: every thread read the same)
  int s0, t0;
  wq_tile(args, wq, cur >> 24, cur & 0xffffff, s0, t0);
  WTile w = wtile_of(args, s_koff, s0, t0);
  load(w, 0);
  for (int j = 0;; ++j) {
    const int nxt = s_next[(j + 1) & 1];
    const bool more = nxt >= 0;
    // The queue's reply is first used after this tile's K loop (the library
    // builds this file without the compiler's wave-level atomic combining,
    // which would wait here).
    int fetched;
    if (tid == 0 && more) fetched = atomicAdd(&ctr[qx], 1);
    WTile w2{};
    if (more) {
      int s2, t2;
      wq_tile(args, wq, nxt >> 24, nxt & 0xffffff, s2, t2);
      w2 = wtile_of(args, s_koff, s2, t2);
    }

    f32x16 acc[2][4];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[nb][mb][q] = 0.0f;

    auto slice = [&]() {
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        bf16x8 af[4], bfr[2];
#pragma unroll
        for (int i = 0; i < 4; ++i) af[i] = *reinterpret_cast<const bf16x8*>(&sTa[fa[i] ^ (kk * 16)]);
#pragma unroll
        for (int i = 0; i < 2; ++i) bfr[i] = *reinterpret_cast<const bf16x8*>(&sTb[fb[i] ^ (kk * 16)]);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int mb = 0; mb < 4; ++mb)
            acc[nb][mb] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[nb], af[mb], acc[nb][mb], 0, 0, 0);
      }
    };
    // Slice kt is staged from registers, then slice kt + 1 (or, for the last
    // slice, the next tile's first) loads while slice kt is multiplied.  The
    // loads are unconditional (an empty range loads nothing), so no wait for
    // them covers stores issued after them.
    store();
    __syncthreads();
    int kt = 0;
    do {
      const bool last = kt + 1 >= w.nk;
      load(last ? w2 : w, last ? 0 : kt + 1);
      if (w.nk > 0) slice();
      __syncthreads();
      if (!last) {
        store();
        __syncthreads();
      }
      ++kt;
    } while (kt < w.nk);
    if (tid == 0 && more)
      s_next[j & 1] =
          fetched < wq_count(args, wq, qx) ? wq_pack(qx, fetched) : take_sync(qx + 1);

    // Epilogue through LDS, 32 rows of the wave's block at a time: the
    // accumulator layout puts one row per lane, so direct stores would send
    // 32-byte pieces of 32 rows per instruction; staged, each store
    // instruction writes four whole 256-byte row pieces.  Each wave stages
    // in its own region (a wave's LDS accesses complete in order, so fences
    // that keep the compiler from reordering them suffice); the barrier at
    // the end keeps the next tile's slice out of regions still read.
    {
      const BgSeg& g = args.seg[w.si];
      float* stage = reinterpret_cast<float*>(sT) + wave * 32 * kWgSP;
      // Stores through a buffer resource over this group's M x ldc output: a
      // row or column outside the output gets an offset past its end, which
      // the hardware drops, so the stores of a round need no branches.
      const int M = g.M, N = g.N, ldc = (int)g.ldc;
      const __amdgpu_buffer_rsrc_t out = __builtin_amdgcn_make_buffer_rsrc(
          static_cast<float*>(g.C) + (int64_t)w.e * g.c_gstride, 0, M * ldc * 4, kBufWord3);
      const int mrow0 = w.m0 + wm * 128, ncol0 = w.n0 + wn * 64;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x16& a = acc[nb][mb];
            *reinterpret_cast<float4*>(
                &stage[(lane & 31) * kWgSP + nb * 32 + 8 * q + 4 * (lane >> 5)]) =
                make_float4(a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]);
          }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int c = ncol0 + 4 * (lane & 15);
        // AUX 2: non-temporal (final gradients: 2.2 GB at the 16B shape
        // would otherwise push the shared operands out of L2)
        auto round = [&](auto aux) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int row = 4 * i + (lane >> 4);
            const int m = mrow0 + mb * 32 + row;
            const u32x4 v = *reinterpret_cast<const u32x4*>(&stage[row * kWgSP + 4 * (lane & 15)]);
            const int off = (m < M && c < N) ? (m * ldc + c) * 4 : kBufDrop;
            __builtin_amdgcn_raw_buffer_store_b128(v, out, off, 0, decltype(aux)::value);
          }
          // all 8 LDS reads in flight at once, then the 8 stores
          __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
          __builtin_amdgcn_sched_group_barrier(0x040, 8, 0);
        };
        if (g.c_stream)
          round(std::integral_constant<int, 2>{});
        else
          round(std::integral_constant<int, 0>{});
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
    }
    __syncthreads();
    if (!more) break;
    w = w2;
  }
}

// SwiGLU backward from kept pre-activations: one wave per row, each lane
// eight consecutive columns per step (eight lanes cover a 64-column block).
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ pre,
    const float* __restrict__ gate, const int32_t* __restrict__ nrows, int64_t rows, int F,
    uint16_t* __restrict__ da, uint16_t* __restrict__ db, uint16_t* __restrict__ gh,
    float* __restrict__ dgp, int ldgp) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t lim = nrows ? (int64_t)*nrows : rows;
  if (r >= lim) return;
  const float g = gate ? gate[r] : 1.0f;
  const int nch = F / 8;
  for (int c0 = 0; c0 < nch; c0 += 64) {
    const int c = c0 + lane;
    float part = 0.0f;
    if (c < nch) {
      const int64_t at = r * F + 8 * c;
      const u32x4 qv = *reinterpret_cast<const u32x4*>(&q[at]);
      const u32x4 av = *reinterpret_cast<const u32x4*>(&pre[r * 2 * F + 8 * c]);
      const u32x4 bv = *reinterpret_cast<const u32x4*>(&pre[r * 2 * F + F + 8 * c]);
      float qf[8], af[8], bf[8];
      unpack4(make_uint2(qv[0], qv[1]), qf);
      unpack4(make_uint2(qv[2], qv[3]), qf + 4);
      unpack4(make_uint2(av[0], av[1]), af);
      unpack4(make_uint2(av[2], av[3]), af + 4);
      unpack4(make_uint2(bv[0], bv[1]), bf);
      unpack4(make_uint2(bv[2], bv[3]), bf + 4);
      float o[3][8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float a = af[j], b = bf[j];
        const float sg = 1.0f / (1.0f + __expf(-a));
        const float sl = a * sg;
        const float dsl = sg * (1.0f + a * (1.0f - sg));
        const float hid = sl * b;
        o[0][j] = g * qf[j] * b * dsl;
        o[1][j] = g * qf[j] * sl;
        o[2][j] = g * hid;
        part += qf[j] * hid;
      }
      uint16_t* dst[3] = {da, db, gh};
#pragma unroll
      for (int w = 0; w < 3; ++w) {
        const uint2 lo = pack4(o[w][0], o[w][1], o[w][2], o[w][3]);
        const uint2 hi = pack4(o[w][4], o[w][5], o[w][6], o[w][7]);
        *reinterpret_cast<u32x4*>(&dst[w][at]) = u32x4{lo.x, lo.y, hi.x, hi.y};
      }
    }
    if (dgp) {
      part += __shfl_xor(part, 1);
      part += __shfl_xor(part, 2);
      part += __shfl_xor(part, 4);
      if ((lane & 7) == 0 && c < nch) dgp[r * ldgp + c / 8] = part;
    }
  }
  if (dgp)
    for (int b = (F + 63) / 64 + lane; b < ldgp; b += 64) dgp[r * ldgp + b] = 0.0f;
}

// One wave per token: its u and dh rows go to each of its grouped rows.
__global__ __launch_bounds__(256) void gather_rows_kernel(
    const int32_t* __restrict__ slot_of, const float* __restrict__ gate,
    const u32x4* __restrict__ u, const u32x4* __restrict__ dh, int64_t T, int k, int nch,
    u32x4* __restrict__ xp, u32x4* __restrict__ dhp, float* __restrict__ gperm,
    int* __restrict__ clear) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (clear && blockIdx.x == 0 && threadIdx.x < kWgQueues) clear[threadIdx.x] = 0;
  if (t >= T) return;
  // slot_of is -1 for an expert id outside [0, n) (the grouping leaves such
  // slots out); they are skipped here and in the kernels below.
  for (int j = lane; j < k; j += 64) {
    const int r = slot_of[t * k + j];
    if (r >= 0) gperm[r] = gate[t * k + j];
  }
  for (int c = lane; c < nch; c += 64) {
    const u32x4 a = u[t * nch + c], b = dh[t * nch + c];
    for (int j = 0; j < k; ++j) {
      const int64_t r = slot_of[t * k + j];
      if (r < 0) continue;
      xp[r * nch + c] = a;
      dhp[r * nch + c] = b;
    }
  }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// One wave per token, four tokens per workgroup; lanes own experts
// lane + 64 q.
__global__ __launch_bounds__(256) void softmax_bwd_kernel(
    const float* __restrict__ lg, int ldlg, int ldl, int64_t T, int n, int k,
    const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ slot_of,
    const float* __restrict__ dgp, int ldgp, const float* __restrict__ f, float alpha,
    uint16_t* __restrict__ dl) {
  __shared__ float sds[4][kMaxExperts];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * 4 + w;
  const bool live = t < T;
  constexpr int Q = kMaxExperts / 64;
  float s[Q];
  float mx = -3.0e38f;
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int i = lane + 64 * q;
    s[q] = (live && i < n) ? lg[t * ldlg + i] : -3.0e38f;
    mx = fmaxf(mx, s[q]);
  }
  mx = wave_max(mx);
  float z = 0.0f;
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int i = lane + 64 * q;
    s[q] = (live && i < n) ? __expf(s[q] - mx) : 0.0f;
    z += s[q];
  }
  z = wave_sum(z);
  const float inv = live ? 1.0f / z : 0.0f;
  const float bal = alpha / (float)T;
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int i = lane + 64 * q;
    s[q] *= inv;
    if (i < n) sds[w][i] = live ? bal * f[i] : 0.0f;
  }
  __syncthreads();
  if (live) {
    for (int j = lane; j < k; j += 64) {
      const int64_t r = slot_of[t * k + j];
      const int e = topk_idx[t * k + j];
      if (r < 0 || e < 0 || e >= n) continue;  // slot left out by the grouping
      float dg = 0.0f;
      for (int p = 0; p < ldgp; ++p) dg += dgp[r * ldgp + p];
      sds[w][e] += dg;  // the kept experts of a token are distinct
    }
  }
  __syncthreads();
  float ds[Q], dot = 0.0f;
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int i = lane + 64 * q;
    ds[q] = i < n ? sds[w][i] : 0.0f;
    dot += s[q] * ds[q];
  }
  dot = wave_sum(dot);
  if (!live) return;
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int i = lane + 64 * q;
    if (i < ldl) dl[t * ldl + i] = i < n ? f32_to_bf16(s[q] * (ds[q] - dot)) : (uint16_t)0;
  }
}

__global__ void slab_sum_kernel(const float4* __restrict__ slabs, int G, int64_t count4,
                                float4* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= count4) return;
  float4 a = slabs[i];
  for (int g = 1; g < G; ++g) {
    const float4 b = slabs[(int64_t)g * count4 + i];
    a.x += b.x;
    a.y += b.y;
    a.z += b.z;
    a.w += b.w;
  }
  out[i] = a;
}

int seg_blocks(BgKind kind, const BgSeg& g) {
  const int nN = (g.N + BN - 1) / BN;
  if (kind == BG_WGRAD) return g.G * ((g.M + WBM - 1) / WBM) * ((g.N + WBN - 1) / WBN);
  if (g.t_off) return g.max_tiles * nN;
  return (int)((g.rows + BM - 1) / BM) * nN;
}

// Compute units of the current device (one persistent weight-gradient
// workgroup each), looked up once per device.
hipError_t cu_count(int* out) {
  static int cached[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (cached[dev] == 0) {
    int v = 0;
    e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (v <= 0) return hipErrorInvalidDevice;
    cached[dev] = v;
  }
  *out = cached[dev];
  return hipSuccess;
}

template <bool BKS, int EPI, bool DUAL, bool PK = false, bool SB = false>
hipError_t launch_t(const BgArgs& args, int grid, hipStream_t s) {
  hipLaunchKernelGGL((bg_kernel<BKS, EPI, DUAL, PK, SB>), dim3(grid), dim3(NT), 0, s, args);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bg(BgKind kind, const BgSeg* segs, int nseg, hipStream_t s, int* work_ctr) {
  if (nseg < 1 || nseg > kBgMaxSeg) return hipErrorInvalidValue;
  BgArgs args{};
  args.nseg = nseg;
  int grid = 0, total = 0;
  for (int i = 0; i < nseg; ++i) {
    args.seg[i] = segs[i];
    args.bound[i] = seg_blocks(kind, segs[i]);
    grid += 8 * ((args.bound[i] + 7) / 8);  // each XCD's share of segment i
    total += args.bound[i];
  }
  if (grid == 0) return hipSuccess;
  if (kind == BG_WGRAD) {
    if (!work_ctr) return hipErrorInvalidValue;
    // the segments with a row-offset table are contiguous and share one
    // table of at most 256 groups
    const int32_t* koff = nullptr;
    int first = -1, last = -1;
    for (int i = 0; i < nseg; ++i) {
      if (!segs[i].koff) continue;
      if (koff && (segs[i].koff != koff || segs[i].G != segs[first].G || last != i - 1))
        return hipErrorInvalidValue;
      if (segs[i].G > kWgMaxGroups) return hipErrorInvalidValue;
      if (!koff) first = i;
      koff = segs[i].koff;
      last = i;
    }
    // each group's output is addressed by a 32-bit buffer offset
    for (int i = 0; i < nseg; ++i)
      if ((int64_t)segs[i].M * segs[i].ldc * 4 >= (int64_t)kBufDrop) return hipErrorInvalidValue;
    int cus = 0;
    const hipError_t e = cu_count(&cus);
    if (e != hipSuccess) return e;
    const int nwg = total < 2 * cus ? total : 2 * cus;  // two per CU
    hipLaunchKernelGGL(wgrad_kernel, dim3(nwg), dim3(NT), 0, s, args, work_ctr);
    return hipGetLastError();
  }
  switch (kind) {
    case BG_LOGITS: return launch_t<false, EPI_F32, false>(args, grid, s);
    case BG_PROJ: return launch_t<true, EPI_BF16, false, false, true>(args, grid, s);
    case BG_SWIGLU: return launch_t<false, EPI_SWIGLU, true, false, true>(args, grid, s);
    case BG_PROJ_PACKED: return launch_t<true, EPI_BF16, false, true, true>(args, grid, s);
    case BG_SWIGLU_PACKED: return launch_t<false, EPI_SWIGLU, true, true, true>(args, grid, s);
    case BG_DU: return launch_t<true, EPI_DU, false>(args, grid, s);
    case BG_WGRAD: break;  // above
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gather_rows(const int32_t* slot_of, const float* topk_gate, const void* u,
                              const void* dh, int64_t T, int k, int d, void* xp, void* dhp,
                              float* gperm, int* clear, hipStream_t s) {
  const int64_t blocks = (T + 3) / 4;
  hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, s, slot_of,
                     topk_gate, static_cast<const u32x4*>(u), static_cast<const u32x4*>(dh), T,
                     k, d / 8, static_cast<u32x4*>(xp), static_cast<u32x4*>(dhp), gperm, clear);
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const uint16_t* q, const uint16_t* pre, const float* gate,
                             const int32_t* nrows, int64_t rows, int F, uint16_t* da,
                             uint16_t* db, uint16_t* gh, float* dgp, int ldgp, hipStream_t s) {
  const int64_t blocks = (rows + 3) / 4;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(swiglu_bwd_kernel, dim3((unsigned)blocks), dim3(256), 0, s, q, pre, gate,
                     nrows, rows, F, da, db, gh, dgp, ldgp);
  return hipGetLastError();
}

hipError_t launch_softmax_bwd(const float* lg, int ldlg, int ldl, int64_t T, int n, int k,
                              const int32_t* topk_idx, const int32_t* slot_of, const float* dgp,
                              int ldgp, const float* f, float alpha, uint16_t* dl, hipStream_t s) {
  const int64_t blocks = (T + 3) / 4;
  hipLaunchKernelGGL(softmax_bwd_kernel, dim3((unsigned)blocks), dim3(256), 0, s, lg, ldlg, ldl,
                     T, n, k, topk_idx, slot_of, dgp, ldgp, f, alpha, dl);
  return hipGetLastError();
}

hipError_t launch_slab_sum(const float* slabs, int G, int64_t count, float* out, hipStream_t s) {
  const int64_t c4 = count / 4;
  const int64_t blocks = (c4 + 255) / 256;
  hipLaunchKernelGGL(slab_sum_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     reinterpret_cast<const float4*>(slabs), G, c4,
                     reinterpret_cast<float4*>(out));
  return hipGetLastError();
}

}  // namespace moe
