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
#include "common.h"

namespace moe {

namespace {

constexpr float kE4M3Max = 448.0f;

// Block scale exponent from the largest magnitude of the block (a
// non-negative binary32 value that is a bf16 value): the biased exponent
// field gives floor(log2 amax) for normal values; subnormal and zero amax
// clamp to -127 either way.
MOE_DEV int mx_exponent(float amax) {
  const int x = static_cast<int>((__float_as_uint(amax) >> 23) & 0xff) - 127 - 8;
  return x < -127 ? -127 : x;
}

// 2^n as binary32 for -126 <= n <= 127.
MOE_DEV float pow2(int n) { return __uint_as_float(static_cast<uint32_t>(n + 127) << 23); }

// E4M3 byte of v * 2^-X; inv = 2^-X. v * inv is exact (a power-of-two scaling
// of a bf16 value) unless it falls below binary32's normal range, where it
// rounds to zero in E4M3 anyway.
MOE_DEV uint32_t e4m3_byte(float v, float inv) {
  const float sv = v * inv;
  const uint32_t sign = (__float_as_uint(sv) >> 24) & 0x80u;
  const float a = fminf(fabsf(sv), kE4M3Max);
  // quantum of a's binade: 2^(e - 3) with e = floor(log2 a), or the
  // subnormal quantum 2^-9 below 2^-6
  const int e = a >= 0x1p-6f ? static_cast<int>(__float_as_uint(a) >> 23) - 127 : -6;
  const float r = fminf(rintf(a * pow2(3 - e)) * pow2(e - 3), kE4M3Max);
  uint32_t code;
  if (r >= 0x1p-6f) {
    const uint32_t rb = __float_as_uint(r);
    code = ((((rb >> 23) & 0xffu) - 127u + 7u) << 3) | ((rb >> 20) & 7u);
  } else {
    code = static_cast<uint32_t>(r * 512.0f);   // m * 2^-9, m = 0..7
  }
  return code | sign;
}

// Scales are stored in groups of four: the word of row r and 128-value column
// group c (the scales of blocks 4c..4c+3) is at byte 4 * (R * c + r).

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
    float v[16];
    float lo[8], hi[8];
    unpack(p[0], lo);
    unpack(p[1], hi);
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[i] = lo[i];
      v[8 + i] = hi[i];
      amax = fmaxf(amax, fmaxf(fabsf(lo[i]), fabsf(hi[i])));
    }
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    const int x = mx_exponent(amax);
    const float inv = pow2(-x);
    V16 out;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t word = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) word |= e4m3_byte(v[4 * w + b], inv) << (8 * b);
      out.w[w] = word;
    }
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

__global__ void __launch_bounds__(256) mx_cols_kernel(const uint16_t* __restrict__ src, int cols, Groups1 gr,
                                                      int col_stride, uint8_t* __restrict__ q,
                                                      uint8_t* __restrict__ s) {
  __shared__ int tile_start[MOE_MAX_EXPERTS + 1];
  __shared__ __attribute__((aligned(16))) uint16_t tile[kQRows * kQLdw];
  const int tid = threadIdx.x;
  const int tiles_c = cols / kQCols;
  const int rt = blockIdx.x / tiles_c, ct = blockIdx.x % tiles_c;

  // group of row-tile rt: tile_start[g] = sum_{h<g} ceil(n_h / 128)
  int g, i;
  if (!gr.offsets) {
    const int per_tiles = (gr.per + kQRows - 1) / kQRows;
    if (per_tiles == 0 || rt >= per_tiles * gr.G) return;
    g = rt / per_tiles;
    i = rt % per_tiles;
  } else {
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
    if (rt >= tile_start[gr.G]) return;
    int lo = 0, hi = gr.G - 1;   // last g with tile_start[g] <= rt
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (tile_start[mid] <= rt) lo = mid;
      else hi = mid - 1;
    }
    g = lo;
    i = rt - tile_start[g];
  }
  int r0, n;
  group_range(gr, g, r0, n);
  // padded column of the group's first row
  const long p_g = gr.offsets ? 128L * tile_start[g]
                              : static_cast<long>(g) * ((gr.per + kQRows - 1) / kQRows) * kQRows;
  const int row_in = i * kQRows;            // first row of the tile within the group
  const int c0 = ct * kQCols;
  // offsets that break the documented contract (decreasing ones) could ask for
  // more padded columns than col_stride holds: such tiles write nothing
  if (p_g + row_in + kQRows > col_stride) return;

  // stage the tile (rows past the group's end read as zeros)
#pragma unroll
  for (int j = 0; j < kQRows * kQCols / 8 / 256; ++j) {
    const int qd = tid + 256 * j;
    const int r = qd / (kQCols / 8), c = qd % (kQCols / 8);
    V16 v = {{0u, 0u, 0u, 0u}};
    if (row_in + r < n)
      v = *reinterpret_cast<const V16*>(src + static_cast<size_t>(r0 + row_in + r) * cols + c0 + c * 8);
    *reinterpret_cast<V16*>(tile + r * kQLdw + c * 8) = v;
  }
  __syncthreads();

  const int c = tid & 63, b = tid >> 6;    // column, block of 32 rows
  float v[32];
  float amax = 0.f;
#pragma unroll
  for (int r = 0; r < 32; ++r) {
    v[r] = bf16_to_f32(tile[(32 * b + r) * kQLdw + c]);
    amax = fmaxf(amax, fabsf(v[r]));
  }
  const int x = mx_exponent(amax);
  const float inv = pow2(-x);
  V16 out[2];
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    uint32_t word = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) word |= e4m3_byte(v[4 * w + k], inv) << (8 * k);
    out[w >> 2].w[w & 3] = word;
  }
  const size_t col = static_cast<size_t>(p_g) + row_in + 32 * b;   // output column of the block
  uint8_t* qp = q + static_cast<size_t>(c0 + c) * col_stride + col;
  reinterpret_cast<V16*>(qp)[0] = out[0];
  reinterpret_cast<V16*>(qp)[1] = out[1];
  // the tile's 128 output columns are one column group: the four block
  // scales of output row c0 + c form one word
  __shared__ uint32_t words[kQCols];
  reinterpret_cast<uint8_t*>(words)[4 * c + b] = static_cast<uint8_t>(x + 127);
  __syncthreads();
  if (tid < kQCols)
    *reinterpret_cast<uint32_t*>(s + 4 * (static_cast<size_t>(cols) * ((p_g + row_in) / kQRows) + c0 + tid)) =
        words[tid];
}

}  // namespace
}  // namespace moe

using namespace moe;

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
