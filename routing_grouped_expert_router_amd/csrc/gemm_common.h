// Grouped-GEMM plumbing shared by the MFMA and the plain FMA kernels: the
// per-op operand mapping and the device-side group-tile scheduler.
#pragma once

#include "common.h"

namespace moe {

// MXFP8 copies of one epilogue output in the two orientations the next GEMMs
// read (the layout of moe_mx_quantize: rows = axis 0, cols = axis 1 with the
// experts as groups); null pointers: not written.
struct MxQOut {
  uint8_t* q_rows;
  uint8_t* s_rows;
  uint8_t* q_cols;
  uint8_t* s_cols;
};

struct GGArgs {
  int op, E, d, F, n_rows, capacity;
  const int32_t* group_offsets;
  void* x_perm;
  void* g;
  void* u;
  void* h;
  void* y_perm;
  void* dy_perm;
  void* dg;
  void* du;
  void* dx_perm;
  void* w_gate;
  void* w_up;
  void* w_down;
  void* dw_gate;
  void* dw_up;
  void* dw_down;
  // weight gradients: the tile split of the launch written by
  // gg_wgrad_split_kernel (kSplitInts ints), or null for the equal-count split
  const int* split;
  // MXFP8 quantised copies of H (FWD_GATE_UP, mxo[0]) or of dG and dU
  // (DGRAD_DOWN, mxo[0] and mxo[1]) written by the epilogue, with the token
  // stride of the column orientation; unused (null) elsewhere
  MxQOut mxo[2];
  int mx_P;
  // weight gradients with K split over ksplit > 1 chunks: binary32 partial
  // sums [ksplit][E][M][NP] (NP = N, or 2N for gate then up), reduced in a
  // fixed order by gg_splitk_reduce_kernel; null and 0 otherwise
  float* partial;
  int ksplit;
};

// Static shape of each op as C[M x N] = sum_k A[m, k] B[k, n] per expert.
template <int OP> struct OpInfo;
template <> struct OpInfo<MOE_GG_FWD_GATE_UP> {
  static constexpr bool kDual = true, kKVar = false, kAKContig = true, kBKContig = false;
};
template <> struct OpInfo<MOE_GG_FWD_DOWN> {
  static constexpr bool kDual = false, kKVar = false, kAKContig = true, kBKContig = false;
};
template <> struct OpInfo<MOE_GG_DGRAD_DOWN> {
  static constexpr bool kDual = false, kKVar = false, kAKContig = true, kBKContig = true;
};
template <> struct OpInfo<MOE_GG_DGRAD_GATE_UP> {
  static constexpr bool kDual = false, kKVar = false, kAKContig = true, kBKContig = true;
};
template <> struct OpInfo<MOE_GG_WGRAD_DOWN> {
  static constexpr bool kDual = false, kKVar = true, kAKContig = false, kBKContig = false;
};
template <> struct OpInfo<MOE_GG_WGRAD_GATE_UP> {
  static constexpr bool kDual = true, kKVar = true, kAKContig = false, kBKContig = false;
};

// Output columns N of an op (per matrix for the dual ops).
inline __host__ __device__ int op_n(int op, int d, int F) {
  switch (op) {
    case MOE_GG_FWD_GATE_UP: return F;
    case MOE_GG_FWD_DOWN: return d;
    case MOE_GG_DGRAD_DOWN: return F;
    case MOE_GG_DGRAD_GATE_UP: return d;
    case MOE_GG_WGRAD_DOWN: return d;
    default: return F;   // WGRAD_GATE_UP
  }
}
// Output rows M of a weight-gradient op.
inline __host__ __device__ int op_wgrad_m(int op, int d, int F) {
  return op == MOE_GG_WGRAD_DOWN ? F : d;
}
// Contraction length of a row-varying op.
inline __host__ __device__ int op_k(int op, int d, int F) {
  switch (op) {
    case MOE_GG_FWD_GATE_UP: return d;
    case MOE_GG_FWD_DOWN: return F;
    case MOE_GG_DGRAD_DOWN: return d;
    default: return 2 * F;   // DGRAD_GATE_UP: [dG | dU] against [Wg ; Wu]
  }
}

// Row range [r0, r0 + n) of expert e, clamped into [0, n_rows].
MOE_DEV void group_rows(const GGArgs& a, int e, int& r0, int& n) {
  if (a.capacity > 0) {
    r0 = e * a.capacity;
    n = a.capacity;
  } else {
    int lo = a.group_offsets[e], hi = a.group_offsets[e + 1];
    lo = lo < 0 ? 0 : (lo > a.n_rows ? a.n_rows : lo);
    hi = hi < lo ? lo : (hi > a.n_rows ? a.n_rows : hi);
    r0 = lo;
    n = hi - lo;
  }
  if (r0 + n > a.n_rows) n = a.n_rows - r0 > 0 ? a.n_rows - r0 : 0;
}

// Workgroups are dispatched round-robin over the 8 XCDs of an MI355X
// (workgroup i runs on XCD i % 8). Map the i-th workgroup of an XCD to the
// i-th tile of a contiguous range of the `tiles` real tiles, so that tiles
// sharing an expert's weights and rows meet in the same L2 and every XCD gets
// an equal share; returns -1 for a workgroup past its XCD's share. Needs
// tiles <= nb (the launch may hold more workgroups than tiles: the grid of a
// row-varying op is sized for the most m-tiles the expert split can need,
// and its real tile count is known on the device only).
MOE_DEV int xcd_tile(int blk, int nb, int tiles) {
  constexpr int kXcd = 8;
  (void)nb;
  const int q = tiles / kXcd, r = tiles % kXcd;
  const int x = blk % kXcd, s = blk / kXcd;
  const int count = q + (x < r ? 1 : 0);
  if (s >= count) return -1;
  return x * q + (x < r ? x : r) + s;
}
MOE_DEV int xcd_remap(int b, int nb) { return xcd_tile(b, nb, nb); }

// Exclusive prefix over the experts of a per-expert count v(e) >= 0, built
// in LDS by one workgroup: out[e] = sum_{h<e} v(h), out[E] = the total
// (E <= MOE_MAX_EXPERTS). Returns the total; every thread of the workgroup
// must call it.
template <int NT, class V>
MOE_DEV int build_expert_prefix(int E, V v, int* out) {
  // per-thread partial sums over a contiguous run of experts
  constexpr int kMaxPer = (MOE_MAX_EXPERTS + NT - 1) / NT;
  const int per = (E + NT - 1) / NT;
  const int e_lo = threadIdx.x * per;
  int loc[kMaxPer];
  int sum = 0;
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) {
    const int t = (i < per && e_lo + i < E) ? v(e_lo + i) : 0;
    loc[i] = t;
    sum += t;
  }
  // exclusive scan of the per-thread sums (NT threads)
  __shared__ int wtot[NT / 64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int incl = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  if (lane == 63) wtot[w] = incl;
  __syncthreads();
  int before = incl - sum;
  for (int i = 0; i < w; ++i) before += wtot[i];
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) {
    if (i < per && e_lo + i < E) out[e_lo + i] = before;
    before += loc[i];
  }
  if (threadIdx.x == NT - 1) out[E] = before;
  __syncthreads();
  return out[E];
}

// Row-varying ops: tile_start[e] = number of BM-row tiles of experts < e
// (tile_start[E] = all m-tiles), from the device-resident group offsets.
template <int BM, int NT>
MOE_DEV int build_tile_prefix(const GGArgs& a, int* tile_start) {
  return build_expert_prefix<NT>(a.E, [&](int e) {
    int r0, n;
    group_rows(a, e, r0, n);
    return (n + BM - 1) / BM;
  }, tile_start);
}

// ------------------------------------------------------------------ weight-gradient tile split
// A weight-gradient launch has one workgroup per tile: every expert has tpe
// = (M/BM)(N/BNO) tiles (numbered expert-major) whose work grows with the
// expert's rows (its K: K steps of BK plus kTileFixed for a tile's prologue
// and epilogue). With experts of about equal size the XCDs split the tiles
// into equal contiguous ranges and each workgroup takes one (xcd_remap). When
// that split leaves one XCD more than kSkew times the mean work, the XCDs
// split the work instead: each takes a contiguous range of tiles holding an
// equal share of it, dealt out to its workgroups in turn (wgrad_tiles). One
// workgroup (gg_wgrad_split_kernel) decides this once per launch and writes
// split[0] = 1 when balancing, split[1 + x] = first tile of XCD x (x = 0..8,
// split[9] = all tiles).
constexpr int kTileFixed = 3;
constexpr float kSkew = 1.25f;
constexpr int kXcdCount = 8;
constexpr int kSplitInts = 2 + kXcdCount;

template <int BK, int NT>
MOE_DEV void wgrad_split(const GGArgs& a, int tpe, int nb, int* scratch, int* split) {
  static_assert(NT >= 2 * kXcdCount + 1, "one thread per XCD check and per boundary");
  auto work = [&](int e) {
    int r0, n;
    group_rows(a, e, r0, n);
    return (n + BK - 1) / BK + kTileFixed;
  };
  build_expert_prefix<NT>(a.E, work, scratch);   // ends with a barrier
  __shared__ long xcd_work[kXcdCount];
  const int T = a.E * tpe;
  const long total = (long)tpe * scratch[a.E];
  auto work_before = [&](int u) -> long {   // work of tiles [0, u)
    if (u >= T) return total;
    const int e = u / tpe;
    return (long)tpe * scratch[e] + (long)(u % tpe) * (scratch[e + 1] - scratch[e]);
  };
  const int tid = threadIdx.x;
  const bool check = nb >= kXcdCount && nb == T;   // the equal-count split of xcd_remap applies
  if (tid < kXcdCount) {
    // XCD tid's work under the equal-count split
    long w = 0;
    if (check) {
      const int q = nb / kXcdCount, r = nb % kXcdCount;
      const int t0 = tid < r ? tid * (q + 1) : r * (q + 1) + (tid - r) * q;
      const int t1 = t0 + q + (tid < r ? 1 : 0);
      w = work_before(t1) - work_before(t0);
    }
    xcd_work[tid] = w;
  } else if (tid < 2 * kXcdCount + 1) {
    // boundary x: the first tile whose work starts at or after x / kXcdCount of the total
    const int x = tid - kXcdCount;
    const long target = total * x / kXcdCount;
    int t;
    if (target <= 0) {
      t = 0;
    } else if (target >= total) {
      t = T;
    } else {
      int lo = 0, hi = a.E - 1;   // last e with tpe * scratch[e] <= target
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((long)tpe * scratch[mid] <= target) lo = mid;
        else hi = mid - 1;
      }
      const long w = scratch[lo + 1] - scratch[lo];
      const long j = (target - (long)tpe * scratch[lo] + w - 1) / w;   // tiles of expert lo before it
      t = j >= tpe ? (lo + 1) * tpe : lo * tpe + (int)j;
    }
    split[1 + x] = t;
  }
  __syncthreads();
  if (tid == 0) {
    long most = 0;
    for (int x = 0; x < kXcdCount; ++x) most = xcd_work[x] > most ? xcd_work[x] : most;
    split[0] = check && (float)most > kSkew * (float)total / kXcdCount ? 1 : 0;
  }
}

// This workgroup's tiles t, t + step, ... (< end) of a weight-gradient
// launch of nb workgroups (one per tile) under the split, or its one tile of
// the equal-count split when the split is null or not balancing. Within its
// XCD's range a workgroup takes every wgs-th tile (wgs = the XCD's
// workgroups): the heaviest tiles of a range then go to different
// workgroups instead of sitting back to back in one. Every tile falls to
// exactly one workgroup.
MOE_DEV void wgrad_tiles(const int* __restrict__ split, int blk, int nb, int& t, int& end, int& step) {
  if (split == nullptr || split[0] == 0) {
    t = xcd_remap(blk, nb);
    end = t + 1;
    step = 1;
    return;
  }
  const int x = blk % kXcdCount, s = blk / kXcdCount;
  const int t0 = split[1 + x], t1 = split[2 + x];
  step = nb / kXcdCount + (x < nb % kXcdCount ? 1 : 0);   // workgroups of this XCD
  t = t0 + s;
  end = t1;
}

// m-tile tm -> (expert, first row, rows), from a built prefix.
template <int BM>
MOE_DEV bool m_tile_of(const GGArgs& a, int tm, const int* tile_start, int& e, int& row0, int& mv) {
  if (tm >= tile_start[a.E]) return false;
  int lo = 0, hi = a.E - 1;   // last e with tile_start[e] <= tm
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tile_start[mid] <= tm) lo = mid;
    else hi = mid - 1;
  }
  e = lo;
  int r0, n;
  group_rows(a, e, r0, n);
  const int mt = tm - tile_start[e];
  row0 = r0 + mt * BM;
  mv = n - mt * BM < BM ? n - mt * BM : BM;
  return true;
}

// Both steps at once (for kernels that launch one workgroup per m-tile slot).
template <int BM, int NT>
MOE_DEV bool find_m_tile(const GGArgs& a, int tm, int* tile_start, int& e, int& row0, int& mv) {
  build_tile_prefix<BM, NT>(a, tile_start);
  return m_tile_of<BM>(a, tm, tile_start, e, row0, mv);
}

// Row-varying ops, expert-grouped order, from a built prefix: linear tile b
// runs over experts in order; inside expert e (with mt_e m-tiles) the tiles
// are ordered n-tile major, m-tile minor, so all m-tiles reading one weight
// slice are adjacent.
template <int BM>
MOE_DEV bool m_tile_grouped(const GGArgs& a, int b, int tilesN, const int* tile_start, int& e, int& row0,
                            int& mv, int& tn) {
  if (b >= tile_start[a.E] * tilesN) return false;
  int lo = 0, hi = a.E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tile_start[mid] * tilesN <= b) lo = mid;
    else hi = mid - 1;
  }
  e = lo;
  const int mt_e = tile_start[e + 1] - tile_start[e];
  const int rel = b - tile_start[e] * tilesN;
  tn = rel / mt_e;
  const int mt = rel % mt_e;
  int r0, n;
  group_rows(a, e, r0, n);
  row0 = r0 + mt * BM;
  mv = n - mt * BM < BM ? n - mt * BM : BM;
  return true;
}

}  // namespace moe
