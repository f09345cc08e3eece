// MXFP8 quantisation (gfx950): bf16 -> E4M3 element bytes + one E8M0 scale
// byte per 32 values, in the two orientations the expert GEMMs need.
//
// The pages name MXFP8 for the feed-forward GEMMs (bigchange.ai pt-BR, "Três
// números, três denominadores") and fix nothing else; the block size, the
// element and scale encodings and the scale rule follow the public OCP
// Microscaling Formats v1.0 specification: X = floor(log2 amax) - 8 (8 is the
// exponent of E4M3's largest normal), clamped to [-127, 127], X = -127 for an
// all-zero block; elements are v * 2^-X rounded to nearest-even, saturated to
// +-448, sign kept. Inputs are finite.
#include "mx_common.h"

#include <algorithm>

namespace moe {

namespace {

// ------------------------------------------------------------------ axis 0
// One thread per 16 values (half a block); the two halves of a block are
// neighbouring lanes and the eight lanes of a 128-value group share one scale
// word, written by the group's first lane. Codes go out as one 16-byte store
// per thread.
__global__ void __launch_bounds__(256) mx_rows_kernel(const uint16_t* __restrict__ src, long n_half, int rows,
                                                      int nb, uint8_t* __restrict__ q, uint8_t* __restrict__ s) {
  const long stride = static_cast<long>(gridDim.x) * 256;   // a multiple of 8: groups stay together
  for (long h = static_cast<long>(blockIdx.x) * 256 + threadIdx.x; h < n_half; h += stride) {
    const V16* p = reinterpret_cast<const V16*>(src + h * 16);
    const V16 lo = p[0], hi = p[1];
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) m = mag_max2(mag_max2(m, lo.w[i]), hi.w[i]);
    m = max2(m, __shfl_xor(m, 1, 64));
    const BlockScale bs = block_scale(max_half(m));
    const int x = bs.x;
    V16 out;
    out.w[0] = encode_quad(lo.w[0], lo.w[1], bs);
    out.w[1] = encode_quad(lo.w[2], lo.w[3], bs);
    out.w[2] = encode_quad(hi.w[0], hi.w[1], bs);
    out.w[3] = encode_quad(hi.w[2], hi.w[3], bs);
    *reinterpret_cast<V16*>(q + h * 16) = out;
    const uint32_t code = static_cast<uint32_t>(x + 127);
    const uint32_t c1 = __shfl_down(code, 2, 64), c2 = __shfl_down(code, 4, 64), c3 = __shfl_down(code, 6, 64);
    if ((h & 7) == 0) {
      const long bl = h >> 1;
      const long r = bl / nb, b = bl % nb;
      *reinterpret_cast<uint32_t*>(s + 4 * (static_cast<size_t>(rows) * (b >> 2) + r)) =
          code | (c1 << 8) | (c2 << 16) | (c3 << 24);
    }
  }
}

// ------------------------------------------------------------------ axis 1
// A workgroup quantises a 128-row x 64-column tile of one group: the tile is
// staged in LDS, then thread (c, b) turns rows 32b..32b+31 of column c into
// 32 code bytes of output row c (two 16-byte stores) and one scale byte.
constexpr int kQRows = 128, kQCols = 64, kQLdw = kQCols + 8;

struct Groups1 {
  const int32_t* offsets;   // device [G+1] or null (equal groups)
  int G, rows, per;         // per: rows of each equal group
};

MOE_DEV void group_range(const Groups1& g, int i, int& r0, int& n) {
  if (!g.offsets) {
    r0 = i * g.per;
    n = g.per;
    return;
  }
  int lo = g.offsets[i], hi = g.offsets[i + 1];
  lo = lo < 0 ? 0 : (lo > g.rows ? g.rows : lo);
  hi = hi < lo ? lo : (hi > g.rows ? g.rows : hi);
  r0 = lo;
  n = hi - lo;
}

// Group and 128-row tile of row-tile index rt (tiles of every group in group
// order, ceil(n_g/128) per group), and the group's first padded column p_g =
// 128 * sum_{h<g} ceil(n_h/128). Every thread of the 256-thread workgroup
// calls it (it synchronises); false: rt is past the last tile.
MOE_DEV bool find_group_tile(const Groups1& gr, int rt, int* tile_start, int& g, int& i, long& p_g) {
  const int tid = threadIdx.x;
  if (!gr.offsets) {
    const int per_tiles = (gr.per + kQRows - 1) / kQRows;
    if (per_tiles == 0 || rt >= per_tiles * gr.G) return false;
    g = rt / per_tiles;
    i = rt % per_tiles;
    p_g = static_cast<long>(g) * per_tiles * kQRows;
    return true;
  }
  constexpr int kMaxPer = (MOE_MAX_EXPERTS + 255) / 256;
  const int per = (gr.G + 255) / 256;
  const int g_lo = tid * per;
  int loc[kMaxPer];
  int sum = 0;
#pragma unroll
  for (int j = 0; j < kMaxPer; ++j) {
    int t = 0;
    if (j < per && g_lo + j < gr.G) {
      int r0, n;
      group_range(gr, g_lo + j, r0, n);
      t = (n + kQRows - 1) / kQRows;
    }
    loc[j] = t;
    sum += t;
  }
  __shared__ int wtot[4];
  const int lane = tid & 63, w = tid >> 6;
  int incl = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wtot[w] = incl;
  __syncthreads();
  int before = incl - sum;
  for (int j = 0; j < w; ++j) before += wtot[j];
#pragma unroll
  for (int j = 0; j < kMaxPer; ++j) {
    if (j < per && g_lo + j < gr.G) tile_start[g_lo + j] = before;
    before += loc[j];
  }
  if (tid == 255) tile_start[gr.G] = before;
  __syncthreads();
  if (rt >= tile_start[gr.G]) return false;
  int lo = 0, hi = gr.G - 1;   // last g with tile_start[g] <= rt
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tile_start[mid] <= rt) lo = mid;
    else hi = mid - 1;
  }
  g = lo;
  i = rt - tile_start[g];
  p_g = 128L * tile_start[g];
  return true;
}

// Stage a tile of TC columns and 128 rows of one group into LDS (rows past the
// group's end read as zeros).
// Row gather of the staged tile: tile row r of group rows [r0 + row_in, ...)
// reads src row `gather[grow] / gk` (the token of permuted row grow) when
// gather is given, else src row grow.
struct RowGather {
  const int32_t* gather;
  int gk;
  int n_src;                // rows of src (a gathered index outside [0, n_src) reads zeros)
};

// Stage a tile of TC columns and 128 rows of one group into LDS (rows past the
// group's end read as zeros). Every load is unconditional (a row past the end
// reads the group's last row of the tile, then zeroed): loads under a per-row
// branch would each be waited for before the next is issued.
template <int TC, int LDW>
MOE_DEV void stage_tile(const uint16_t* __restrict__ src, int cols, int r0, int n, int row_in, int c0,
                        uint16_t* tile) {
  constexpr int CH = TC / 8;   // 16-byte chunks per row
  constexpr int NJ = kQRows * CH / 256;
  V16 v[NJ];
  const int last = n - row_in - 1;   // >= 0: the tile holds at least one row
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int qd = threadIdx.x + 256 * j;
    const int r = qd / CH, c = qd % CH;
    v[j] = *reinterpret_cast<const V16*>(src + static_cast<size_t>(r0 + row_in + min(r, last)) * cols + c0 + c * 8);
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int qd = threadIdx.x + 256 * j;
    const int r = qd / CH, c = qd % CH;
    *reinterpret_cast<V16*>(tile + r * LDW + c * 8) = keep_if(r <= last, v[j]);
  }
}

// Column (transposed) quantisation of the tile's columns [c_lo, c_lo + 64):
// thread (c, b) turns rows 32b..32b+31 of column c into 32 code bytes of output
// row c0 + c and one scale byte; the four scales of a column form one word.
template <int LDW>
MOE_DEV void cols_part(const uint16_t* tile, int c_lo, int c0, int cols, long p_g, int row_in, int col_stride,
                       uint8_t* __restrict__ q, uint8_t* __restrict__ s, uint32_t* words) {
  const int tid = threadIdx.x;
  const int c = c_lo + (tid & 63), b = tid >> 6;
  uint32_t w[16];
#pragma unroll
  for (int r = 0; r < 16; ++r)
    w[r] = static_cast<uint32_t>(tile[(32 * b + 2 * r) * LDW + c]) |
           static_cast<uint32_t>(tile[(32 * b + 2 * r + 1) * LDW + c]) << 16;
  V16 out[2];
  const uint32_t code = quantize_block_bf16(w, out);
  const size_t col = static_cast<size_t>(p_g) + row_in + 32 * b;   // output column of the block
  uint8_t* qp = q + static_cast<size_t>(c0 + c) * col_stride + col;
  reinterpret_cast<V16*>(qp)[0] = out[0];
  reinterpret_cast<V16*>(qp)[1] = out[1];
  reinterpret_cast<uint8_t*>(words)[4 * (c - c_lo) + b] = static_cast<uint8_t>(code);
  __syncthreads();
  if (tid < 64)
    *reinterpret_cast<uint32_t*>(s + 4 * (static_cast<size_t>(cols) * ((p_g + row_in) / kQRows) + c0 + c_lo + tid)) =
        words[tid];
  __syncthreads();
}

__global__ void __launch_bounds__(256) mx_cols_kernel(const uint16_t* __restrict__ src, int cols, Groups1 gr,
                                                      int col_stride, uint8_t* __restrict__ q,
                                                      uint8_t* __restrict__ s) {
  __shared__ int tile_start[MOE_MAX_EXPERTS + 1];
  __shared__ __attribute__((aligned(16))) uint16_t tile[kQRows * kQLdw];
  __shared__ uint32_t words[64];
  const int tiles_c = cols / kQCols;
  const int rt = blockIdx.x / tiles_c, ct = blockIdx.x % tiles_c;
  int g, i;
  long p_g;
  if (!find_group_tile(gr, rt, tile_start, g, i, p_g)) return;
  int r0, n;
  group_range(gr, g, r0, n);
  const int row_in = i * kQRows;            // first row of the tile within the group
  const int c0 = ct * kQCols;
  // offsets that break the documented contract (decreasing ones) could ask for
  // more padded columns than col_stride holds: such tiles write nothing
  if (p_g + row_in + kQRows > col_stride) return;
  stage_tile<kQCols, kQLdw>(src, cols, r0, n, row_in, c0, tile);
  __syncthreads();
  cols_part<kQLdw>(tile, 0, c0, cols, p_g, row_in, col_stride, q, s, words);
}

// ------------------------------------------------------------------ both
// One pass, both orientations: a 128-row x 128-column tile of one group is
// staged once; the column part (cols_quads) writes the transposed codes, and
// the row part quantises each valid row's 128 values (four blocks, one scale
// word) into the row-oriented output. Workgroups are persistent: each takes a
// contiguous run of tiles and holds the next tile's loads in registers while
// it quantises the current one, so load latency overlaps the work.
constexpr int kBCols = 128, kBLdw = kBCols + 8;
constexpr int kBChunks = kQRows * kBCols / 8 / 256;   // 16-byte loads per thread per tile

// Tiles per group prefix: tile_start[g] = sum_{h<g} ceil(n_h/128) (device
// offsets); returns the number of row tiles. Every thread calls it.
// grp_rows (optional, 2 G ints in LDS): each group's clamped first row and row
// count, so that the tile loop reads group ranges from LDS, not memory.
MOE_DEV int build_tile_prefix(const Groups1& gr, int* tile_start, int* grp_rows = nullptr) {
  if (!gr.offsets) return gr.G * ((gr.per + kQRows - 1) / kQRows);
  const int tid = threadIdx.x;
  constexpr int kMaxPer = (MOE_MAX_EXPERTS + 255) / 256;
  const int per = (gr.G + 255) / 256;
  const int g_lo = tid * per;
  int loc[kMaxPer];
  int sum = 0;
#pragma unroll
  for (int j = 0; j < kMaxPer; ++j) {
    int t = 0;
    if (j < per && g_lo + j < gr.G) {
      int r0, n;
      group_range(gr, g_lo + j, r0, n);
      t = (n + kQRows - 1) / kQRows;
      if (grp_rows) {
        grp_rows[2 * (g_lo + j)] = r0;
        grp_rows[2 * (g_lo + j) + 1] = n;
      }
    }
    loc[j] = t;
    sum += t;
  }
  __shared__ int wtot[4];
  const int lane = tid & 63, w = tid >> 6;
  int incl = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wtot[w] = incl;
  __syncthreads();
  int before = incl - sum;
  for (int j = 0; j < w; ++j) before += wtot[j];
#pragma unroll
  for (int j = 0; j < kMaxPer; ++j) {
    if (j < per && g_lo + j < gr.G) tile_start[g_lo + j] = before;
    before += loc[j];
  }
  if (tid == 255) tile_start[gr.G] = before;
  __syncthreads();
  return tile_start[gr.G];
}

// Group g, tile i within it and p_g of row tile rt < total row tiles.
MOE_DEV void lookup_tile(const Groups1& gr, const int* tile_start, int rt, int& g, int& i, long& p_g) {
  if (!gr.offsets) {
    const int per_tiles = (gr.per + kQRows - 1) / kQRows;
    g = rt / per_tiles;
    i = rt % per_tiles;
    p_g = static_cast<long>(g) * per_tiles * kQRows;
    return;
  }
  int lo = 0, hi = gr.G - 1;   // last g with tile_start[g] <= rt
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tile_start[mid] <= rt) lo = mid;
    else hi = mid - 1;
  }
  g = lo;
  i = rt - tile_start[g];
  p_g = 128L * tile_start[g];
}

struct BothTile {
  int r0, n, row_in, c0;
  long p_g;
  bool skip;   // would write past col_stride (offsets that break the contract)
};

// Tile j of the row-tile-major order: row tile j / tiles_c, column tile
// j % tiles_c, so a workgroup's consecutive tiles read the same 128 source
// rows a column tile further each time (whole rows close together in time,
// which suits DRAM better than revisiting each row once per column pass; every
// transposed piece is a whole aligned 128-byte line either way).
MOE_DEV BothTile both_tile(const Groups1& gr, const int* tile_start, const int* grp_rows, int total_rt,
                           int col_stride, long j, int tiles_c) {
  BothTile t;
  int g, i;
  lookup_tile(gr, tile_start, static_cast<int>(j / tiles_c), g, i, t.p_g);
  if (gr.offsets) {
    t.r0 = grp_rows[2 * g];
    t.n = grp_rows[2 * g + 1];
  } else {
    group_range(gr, g, t.r0, t.n);
  }
  t.row_in = i * kQRows;
  t.c0 = static_cast<int>(j % tiles_c) * kBCols;
  t.skip = t.p_g + t.row_in + kQRows > col_stride;
  return t;
}

// The tile's 16-byte chunks of this thread. Rows past the group's end, and
// gathered rows outside the source, read as zeros: every load is issued
// unconditionally (a missing row reads a valid one) and `valid` records
// which chunks keep their value (applied when the chunks go to LDS). With a
// gather, the eight row indices are loaded first, then the eight chunks.
template <bool GATHER>
MOE_DEV void fetch_tile(const uint16_t* __restrict__ src, int cols, const BothTile& t, RowGather rg,
                        V16 (&v)[kBChunks], uint32_t& valid) {
  constexpr int CH = kBCols / 8;
  const int last = t.n - t.row_in - 1;   // >= 0: the tile holds at least one row
  long srow[kBChunks];
  valid = 0;
#pragma unroll
  for (int j = 0; j < kBChunks; ++j) {
    const int r = (threadIdx.x + 256 * j) / CH;
    srow[j] = static_cast<long>(t.r0) + t.row_in + min(r, last);
    if (r <= last) valid |= 1u << j;
  }
  if constexpr (GATHER) {
    int slot[kBChunks];
#pragma unroll
    for (int j = 0; j < kBChunks; ++j) slot[j] = rg.gather[srow[j]];
#pragma unroll
    for (int j = 0; j < kBChunks; ++j) {
      const long sr = slot[j] >= 0 ? slot[j] / rg.gk : -1;
      const bool ok = sr >= 0 && sr < rg.n_src;
      if (!ok) valid &= ~(1u << j);
      srow[j] = ok ? sr : 0;
    }
  }
#pragma unroll
  for (int j = 0; j < kBChunks; ++j) {
    const int c = (threadIdx.x + 256 * j) % CH;
    v[j] = *reinterpret_cast<const V16*>(src + static_cast<size_t>(srow[j]) * cols + t.c0 + c * 8);
  }
}

// Column part of the two-orientation pass: thread (quad of 4 columns, block b,
// half h) reads 16 rows x 4 columns of the staged tile with 8-byte LDS reads
// (a quarter of the LDS reads of cols_part), the two halves of a block combine
// their column maxima with one lane shuffle, each thread encodes its 16 rows
// of 4 columns (one 16-byte store per output row) and the first half stores
// the block's four scale bytes.
MOE_DEV void cols_quads(const uint16_t* tile, int c0, int cols, long p_g, int row_in, int col_stride,
                        uint8_t* __restrict__ q, uint8_t* __restrict__ s) {
  const int tid = threadIdx.x;
  const int h = tid & 1, b = (tid >> 1) & 3, qd = tid >> 3;   // 32 quads x 4 blocks x 2 halves
  // words of tile rows 32b + 16h + r: columns (4qd, 4qd+1) and (4qd+2, 4qd+3)
  uint32_t w01[16], w23[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const uint2 w = *reinterpret_cast<const uint2*>(tile + (32 * b + 16 * h + r) * kBLdw + 4 * qd);
    w01[r] = w.x;
    w23[r] = w.y;
  }
  uint32_t m01 = 0, m23 = 0;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    m01 = mag_max2(m01, w01[r]);
    m23 = mag_max2(m23, w23[r]);
  }
  m01 = max2(m01, __shfl_xor(m01, 1, 64));
  m23 = max2(m23, __shfl_xor(m23, 1, 64));
  const size_t col = static_cast<size_t>(p_g) + row_in + 32 * b + 16 * h;   // first token column
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t m = j < 2 ? m01 : m23;
    const BlockScale bs = block_scale(j & 1 ? m >> 16 : m & 0xffffu);
    // rows 2i, 2i+1 of column j side by side: the low (j even) or high halves
    const uint32_t sel = j & 1 ? 0x07060302u : 0x05040100u;
    const uint32_t* wj = j < 2 ? w01 : w23;
    V16 out;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      out.w[q] = encode_quad(__builtin_amdgcn_perm(wj[4 * q + 1], wj[4 * q], sel),
                             __builtin_amdgcn_perm(wj[4 * q + 3], wj[4 * q + 2], sel), bs);
    const int c = 4 * qd + j;
    *reinterpret_cast<V16*>(q + static_cast<size_t>(c0 + c) * col_stride + col) = out;
    if (h == 0)
      s[4 * (static_cast<size_t>(cols) * ((p_g + row_in) / kQRows) + c0 + c) + b] = static_cast<uint8_t>(bs.x + 127);
  }
}

template <bool GATHER>
__global__ void __launch_bounds__(256) mx_both_kernel(const uint16_t* __restrict__ src, int rows, int cols,
                                                      Groups1 gr, int col_stride, uint8_t* __restrict__ q_rows,
                                                      uint8_t* __restrict__ s_rows, uint8_t* __restrict__ q_cols,
                                                      uint8_t* __restrict__ s_cols, RowGather rg) {
  __shared__ int tile_start[MOE_MAX_EXPERTS + 1];
  __shared__ int grp_rows[2 * MOE_MAX_EXPERTS];
  __shared__ __attribute__((aligned(16))) uint16_t tile[kQRows * kBLdw];
  const int tid = threadIdx.x;
  const int tiles_c = cols / kBCols;
  const int total_rt = build_tile_prefix(gr, tile_start, grp_rows);
  const long total = static_cast<long>(total_rt) * tiles_c;
  // a contiguous run of tiles per workgroup
  const long per = (total + gridDim.x - 1) / gridDim.x;
  long b = blockIdx.x * per;
  const long b_end = b + per < total ? b + per : total;
  V16 pre[kBChunks];
  uint32_t valid = 0;
  if (b < b_end) fetch_tile<GATHER>(src, cols, both_tile(gr, tile_start, grp_rows, total_rt, col_stride, b, tiles_c), rg, pre, valid);
  for (; b < b_end; ++b) {
    const BothTile t = both_tile(gr, tile_start, grp_rows, total_rt, col_stride, b, tiles_c);
    if (!t.skip) {
      constexpr int CH = kBCols / 8;
#pragma unroll
      for (int j = 0; j < kBChunks; ++j) {
        const int qd = tid + 256 * j;
        *reinterpret_cast<V16*>(tile + (qd / CH) * kBLdw + (qd % CH) * 8) = keep_if((valid >> j) & 1u, pre[j]);
      }
    }
    __syncthreads();
    const long nb = b + 1;
    if (nb < b_end)
      fetch_tile<GATHER>(src, cols, both_tile(gr, tile_start, grp_rows, total_rt, col_stride, nb, tiles_c), rg, pre, valid);
    if (!t.skip) {
      const int r0 = t.r0, n = t.n, row_in = t.row_in, c0 = t.c0;
      // rows: thread (r, h) quantises blocks 2h, 2h+1 (64 values) of tile row r
      {
        const int r = tid >> 1, h = tid & 1;
        uint32_t w[32];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const V16 t8 = *reinterpret_cast<const V16*>(tile + r * kBLdw + 64 * h + 8 * k);
#pragma unroll
          for (int m = 0; m < 4; ++m) w[4 * k + m] = t8.w[m];
        }
        V16 out[2][2];
        const uint32_t c_lo = quantize_block_bf16(w, out[0]);
        const uint32_t c_hi = quantize_block_bf16(w + 16, out[1]);
        const uint32_t pair = c_lo | (c_hi << 8);
        const uint32_t other = __shfl_xor(pair, 1, 64);
        if (row_in + r < n) {
          const size_t grow = static_cast<size_t>(r0) + row_in + r;
          V16* qp = reinterpret_cast<V16*>(q_rows + grow * cols + c0 + 64 * h);
          qp[0] = out[0][0];
          qp[1] = out[0][1];
          qp[2] = out[1][0];
          qp[3] = out[1][1];
          if (h == 0)
            *reinterpret_cast<uint32_t*>(s_rows + 4 * (static_cast<size_t>(rows) * (c0 / kBCols) + grow)) =
                pair | (other << 16);
        }
      }
      cols_quads(tile, c0, cols, t.p_g, row_in, col_stride, q_cols, s_cols);
    }
    __syncthreads();
  }
}

}  // namespace
}  // namespace moe

using namespace moe;

namespace {
// persistent workgroups of the two-orientation quantiser: as many as are
// resident at once (three per CU at its register use)
constexpr long kBothGrid = 256 * 3;
}  // namespace

extern "C" int moe_mx_col_stride(int rows, int n_groups) {
  if (rows < 0 || n_groups < 1) return -1;
  const long v = 128L * ((rows + 127L) / 128 + n_groups);
  return v < (1L << 31) ? static_cast<int>(v) : -1;
}

extern "C" int moe_mx_quantize(const void* src, int rows, int cols, int axis, const int32_t* group_offsets,
                               int n_groups, int col_stride, void* q, void* s, hipStream_t stream) {
  MOE_CHECK_ARG(rows >= 0 && cols > 0 && (axis == 0 || axis == 1));
  if (axis == 0) {
    MOE_CHECK_ARG(cols % 128 == 0 && group_offsets == nullptr && col_stride == 0);
    if (rows == 0) return MOE_OK;
    MOE_CHECK_ARG(src && q && s && aligned16(src) && aligned16(q) && aligned4(s));
    const long n_half = static_cast<long>(rows) * (cols / 16);
    MOE_CHECK_SUPPORTED(n_half < (1L << 40));
    long blocks = (n_half + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    mx_rows_kernel<<<static_cast<int>(blocks), 256, 0, stream>>>(
        static_cast<const uint16_t*>(src), n_half, rows, cols / 32, static_cast<uint8_t*>(q),
        static_cast<uint8_t*>(s));
    return launch_status();
  }
  MOE_CHECK_ARG(cols % kQCols == 0 && n_groups >= 1 && col_stride > 0 && col_stride % 128 == 0);
  MOE_CHECK_SUPPORTED(n_groups <= MOE_MAX_EXPERTS);
  Groups1 gr{group_offsets, n_groups, rows, 0};
  long need;
  if (group_offsets) {
    need = 128L * ((rows + 127L) / 128 + n_groups);
  } else {
    MOE_CHECK_ARG(rows % n_groups == 0);
    gr.per = rows / n_groups;
    need = static_cast<long>(n_groups) * ((gr.per + 127L) / 128) * 128;
  }
  MOE_CHECK_ARG(col_stride >= need);
  MOE_CHECK_SUPPORTED(static_cast<long>(cols) * col_stride < (1L << 40));
  if (rows == 0) return MOE_OK;
  MOE_CHECK_ARG(src && q && s && aligned16(src) && aligned16(q) && aligned4(s));
  const long row_tiles = group_offsets ? (rows + kQRows - 1) / kQRows + n_groups
                                       : static_cast<long>(n_groups) * ((gr.per + kQRows - 1) / kQRows);
  const long grid = row_tiles * (cols / kQCols);
  MOE_CHECK_SUPPORTED(grid < (1L << 31));
  mx_cols_kernel<<<static_cast<int>(grid), 256, 0, stream>>>(static_cast<const uint16_t*>(src), cols, gr,
                                                             col_stride, static_cast<uint8_t*>(q),
                                                             static_cast<uint8_t*>(s));
  return launch_status();
}

extern "C" int moe_mx_quantize_both(const void* src, int rows, int cols, const int32_t* group_offsets,
                                    int n_groups, int col_stride, void* q_rows, void* s_rows, void* q_cols,
                                    void* s_cols, hipStream_t stream) {
  MOE_CHECK_ARG(rows >= 0 && cols > 0 && cols % 128 == 0);
  MOE_CHECK_ARG(n_groups >= 1 && col_stride > 0 && col_stride % 128 == 0);
  MOE_CHECK_SUPPORTED(n_groups <= MOE_MAX_EXPERTS);
  Groups1 gr{group_offsets, n_groups, rows, 0};
  long need;
  if (group_offsets) {
    need = 128L * ((rows + 127L) / 128 + n_groups);
  } else {
    MOE_CHECK_ARG(rows % n_groups == 0);
    gr.per = rows / n_groups;
    need = static_cast<long>(n_groups) * ((gr.per + 127L) / 128) * 128;
  }
  MOE_CHECK_ARG(col_stride >= need);
  MOE_CHECK_SUPPORTED(static_cast<long>(cols) * col_stride < (1L << 40) && static_cast<long>(rows) * cols < (1L << 40));
  if (rows == 0) return MOE_OK;
  MOE_CHECK_ARG(src && q_rows && s_rows && q_cols && s_cols && aligned16(src) && aligned16(q_rows) &&
                aligned16(q_cols) && aligned4(s_rows) && aligned4(s_cols));
  const long row_tiles = group_offsets ? (rows + kQRows - 1) / kQRows + n_groups
                                       : static_cast<long>(n_groups) * ((gr.per + kQRows - 1) / kQRows);
  const long grid = std::min(row_tiles * (cols / kBCols), kBothGrid);
  mx_both_kernel<false><<<static_cast<int>(grid), 256, 0, stream>>>(
      static_cast<const uint16_t*>(src), rows, cols, gr, col_stride, static_cast<uint8_t*>(q_rows),
      static_cast<uint8_t*>(s_rows), static_cast<uint8_t*>(q_cols), static_cast<uint8_t*>(s_cols),
      RowGather{nullptr, 1, 0});
  return launch_status();
}

extern "C" int moe_permute_mx(const void* x, int T, int d, int k, const int32_t* src_slot,
                              const int32_t* group_offsets, int E, int n_rows, int col_stride, void* q_rows,
                              void* s_rows, void* q_cols, void* s_cols, hipStream_t stream) {
  MOE_CHECK_ARG(T >= 0 && d > 0 && d % 128 == 0 && k >= 1 && E >= 1 && n_rows >= 0);
  MOE_CHECK_SUPPORTED(k <= MOE_MAX_TOPK && E <= MOE_MAX_EXPERTS && static_cast<long>(T) * k < (1L << 31));
  MOE_CHECK_ARG(static_cast<long>(n_rows) == static_cast<long>(T) * k);   // dropless rows only
  MOE_CHECK_ARG(col_stride > 0 && col_stride % 128 == 0 && col_stride >= 128L * ((n_rows + 127L) / 128 + E));
  MOE_CHECK_SUPPORTED(static_cast<long>(d) * col_stride < (1L << 40) && static_cast<long>(n_rows) * d < (1L << 40));
  if (n_rows == 0) return MOE_OK;
  MOE_CHECK_ARG(x && src_slot && group_offsets && aligned16(x));
  MOE_CHECK_ARG(q_rows && s_rows && q_cols && s_cols && aligned16(q_rows) && aligned16(q_cols) &&
                aligned4(s_rows) && aligned4(s_cols));
  Groups1 gr{group_offsets, E, n_rows, 0};
  const long grid = std::min(((n_rows + kQRows - 1) / kQRows + E) * static_cast<long>(d / kBCols), kBothGrid);
  mx_both_kernel<true><<<static_cast<int>(grid), 256, 0, stream>>>(
      static_cast<const uint16_t*>(x), n_rows, d, gr, col_stride, static_cast<uint8_t*>(q_rows),
      static_cast<uint8_t*>(s_rows), static_cast<uint8_t*>(q_cols), static_cast<uint8_t*>(s_cols),
      RowGather{src_slot, k, T});
  return launch_status();
}
