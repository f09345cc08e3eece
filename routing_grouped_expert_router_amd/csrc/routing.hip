// Router GEMM, top-k gate, GPU-resident routing metadata, and the router's
// backward (gfx950). See include/moe.h for the contract of each entry point.
#include "common.h"

namespace moe {

// ============================================================== router GEMM
// logits[t, e] = sum_i x[t, i] w_r[i, e]. Memory-bound on x (E is small): one
// wave streams TOK tokens' rows with 16-byte loads while w_r (d x E, a few
// tens of KB) stays in L1/L2; experts are handled 8 at a time.
constexpr int kRouterTok = 4;
constexpr int kRouterEC = 8;

// wide: E is a multiple of 8 and w_r 16-byte aligned, so each row's group of
// eight experts is read as 16-byte vectors
template <typename T>
__global__ void __launch_bounds__(256) router_gemm_kernel(const T* __restrict__ x,
                                                          const T* __restrict__ w_r, int T_,
                                                          int d, int E, bool wide,
                                                          float* __restrict__ logits) {
  constexpr int V = kVec<T>;
  const int lane = threadIdx.x & 63;
  const int wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int t0 = wave * kRouterTok;
  if (t0 >= T_) return;
  const int nvec = d / V;
  for (int e0 = 0; e0 < E; e0 += kRouterEC) {
    float acc[kRouterTok][kRouterEC];
#pragma unroll
    for (int a = 0; a < kRouterTok; ++a)
#pragma unroll
      for (int b = 0; b < kRouterEC; ++b) acc[a][b] = 0.f;
    for (int c = lane; c < nvec; c += 64) {
      float xv[kRouterTok][V];
#pragma unroll
      for (int a = 0; a < kRouterTok; ++a) {
        if (t0 + a < T_) {
          V16 v = *reinterpret_cast<const V16*>(x + (size_t)(t0 + a) * d + (size_t)c * V);
          unpack(v, xv[a]);
        } else {
#pragma unroll
          for (int i = 0; i < V; ++i) xv[a][i] = 0.f;
        }
      }
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const T* wrow = w_r + (size_t)(c * V + i) * E + e0;
        float wv[kRouterEC];
        if (wide) {
          // the eight weights of this row as 16-byte loads
#pragma unroll
          for (int h = 0; h < kRouterEC / V; ++h) {
            float f[V];
            unpack(reinterpret_cast<const V16*>(wrow)[h], f);
#pragma unroll
            for (int m = 0; m < V; ++m) wv[h * V + m] = f[m];
          }
        } else {
#pragma unroll
          for (int b = 0; b < kRouterEC; ++b) wv[b] = (e0 + b < E) ? Elem<T>::load(wrow, b) : 0.f;
        }
#pragma unroll
        for (int b = 0; b < kRouterEC; ++b)
#pragma unroll
          for (int a = 0; a < kRouterTok; ++a) acc[a][b] = fmaf(xv[a][i], wv[b], acc[a][b]);
      }
    }
#pragma unroll
    for (int a = 0; a < kRouterTok; ++a)
#pragma unroll
      for (int b = 0; b < kRouterEC; ++b) acc[a][b] = wave_sum(acc[a][b]);
#pragma unroll
    for (int a = 0; a < kRouterTok; ++a)
#pragma unroll
      for (int b = 0; b < kRouterEC; ++b)
        if (lane == a * kRouterEC + b && t0 + a < T_ && e0 + b < E)
          logits[(size_t)(t0 + a) * E + e0 + b] = acc[a][b];
  }
}

// The same product for bf16 with w_r staged in LDS (E a multiple of 8 and
// d x E small enough): every wave otherwise re-reads each 8-row group of w_r
// from L1, 64 separate lines per load instruction, which made w_r rather than
// x set the rate. Rows are stored in groups of eight with 16 bytes of padding
// after each group, so the 16 lanes of a read phase, which read the same
// expert columns of 16 consecutive groups, hit 16 distinct bank quads. The
// arithmetic and its order are those of router_gemm_kernel.
__host__ __device__ constexpr int router_lds_group_bytes(int E) { return 8 * E * 2 + 16; }

__global__ void __launch_bounds__(256) router_gemm_lds_kernel(const uint16_t* __restrict__ x,
                                                              const uint16_t* __restrict__ w_r, int T_,
                                                              int d, int E, float* __restrict__ logits) {
  extern __shared__ __attribute__((aligned(16))) uint8_t w_lds[];
  constexpr int V = 8;
  const int gb = router_lds_group_bytes(E);
  // stage w_r: 16-byte pieces (8 experts of one row; E % 8 == 0)
  const int pieces = d * E / 8;
  for (int j = threadIdx.x; j < pieces; j += blockDim.x) {
    const int row = j * 8 / E, col = j * 8 % E;
    *reinterpret_cast<V16*>(w_lds + (row >> 3) * gb + (row & 7) * E * 2 + col * 2) =
        reinterpret_cast<const V16*>(w_r)[j];
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int nvec = d / V;
  // each wave takes groups of kRouterTok tokens, grid-strided (one group per
  // wave at the launch's grid)
  const int waves = gridDim.x * (blockDim.x >> 6);
  for (int g = (blockIdx.x * blockDim.x + threadIdx.x) >> 6; g * kRouterTok < T_; g += waves) {
    const int t0 = g * kRouterTok;
    for (int e0 = 0; e0 < E; e0 += kRouterEC) {
      float acc[kRouterTok][kRouterEC];
#pragma unroll
      for (int a = 0; a < kRouterTok; ++a)
#pragma unroll
        for (int b = 0; b < kRouterEC; ++b) acc[a][b] = 0.f;
      for (int c = lane; c < nvec; c += 64) {
        float xv[kRouterTok][V];
#pragma unroll
        for (int a = 0; a < kRouterTok; ++a) {
          if (t0 + a < T_) {
            V16 v = *reinterpret_cast<const V16*>(x + (size_t)(t0 + a) * d + (size_t)c * V);
            unpack(v, xv[a]);
          } else {
#pragma unroll
            for (int i = 0; i < V; ++i) xv[a][i] = 0.f;
          }
        }
        const uint8_t* grp = w_lds + c * gb + e0 * 2;   // rows c*8 .. c*8+7
#pragma unroll
        for (int i = 0; i < V; ++i) {
          float wv[kRouterEC];
          unpack(*reinterpret_cast<const V16*>(grp + i * E * 2), wv);
#pragma unroll
          for (int b = 0; b < kRouterEC; ++b)
#pragma unroll
            for (int a = 0; a < kRouterTok; ++a) acc[a][b] = fmaf(xv[a][i], wv[b], acc[a][b]);
        }
      }
#pragma unroll
      for (int a = 0; a < kRouterTok; ++a)
#pragma unroll
        for (int b = 0; b < kRouterEC; ++b) acc[a][b] = wave_sum(acc[a][b]);
#pragma unroll
      for (int a = 0; a < kRouterTok; ++a)
#pragma unroll
        for (int b = 0; b < kRouterEC; ++b)
          if (lane == a * kRouterEC + b && t0 + a < T_ && e0 + b < E)
            logits[(size_t)(t0 + a) * E + e0 + b] = acc[a][b];
    }
  }
}

// ============================================================== top-k gate
// Order-preserving key of a binary32 value (-0 first mapped to +0), with the
// expert id in the low word so that equal logits prefer the lower id.
MOE_DEV uint64_t gate_key(float f, int e) {
  if (f == 0.0f) f = 0.0f;
  uint32_t u = __float_as_uint(f);
  uint32_t k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<uint64_t>(k) << 32) | static_cast<uint32_t>(0xffffffffu - static_cast<uint32_t>(e));
}
MOE_DEV float key_value(uint64_t key) {
  uint32_t k = static_cast<uint32_t>(key >> 32);
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}
MOE_DEV int key_expert(uint64_t key) {
  return static_cast<int>(0xffffffffu - static_cast<uint32_t>(key));
}

// L lanes share one token and hold P logits each (expert e = g + L*p for lane
// g of the group). Each of the k rounds is a max-reduction over the group.
template <int L, int P>
__global__ void __launch_bounds__(256) route_kernel(const float* __restrict__ logits, int T_, int E,
                                                    int k, int32_t* __restrict__ topk_idx,
                                                    float* __restrict__ topk_w) {
  const int gtid = blockIdx.x * blockDim.x + threadIdx.x;
  const int t = gtid / L;
  const int g = threadIdx.x % L;
  const bool live = t < T_;
  uint64_t key[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int e = g + L * p;
    key[p] = (live && e < E) ? gate_key(logits[(size_t)t * E + e], e) : 0ull;
  }
  float sel_l[MOE_MAX_TOPK];
  int sel_e[MOE_MAX_TOPK];
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j) {
    if (j >= k) break;
    uint64_t best = 0;
#pragma unroll
    for (int p = 0; p < P; ++p) best = key[p] > best ? key[p] : best;
#pragma unroll
    for (int o = L / 2; o > 0; o >>= 1) {
      const uint64_t other = __shfl_xor(best, o, 64);
      best = other > best ? other : best;
    }
    const int e = key_expert(best);
    sel_e[j] = e;
    sel_l[j] = key_value(best);
    if (e % L == g) {
#pragma unroll
      for (int p = 0; p < P; ++p)
        if (p == e / L) key[p] = 0ull;
    }
  }
  if (!live) return;
  const float m = sel_l[0];
  float den = 0.f;
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j)
    if (j < k) den += expf(sel_l[j] - m);
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j) {
    if (j < k && g == j % L && (j / L) == 0) {
      topk_idx[(size_t)t * k + j] = sel_e[j];
      topk_w[(size_t)t * k + j] = expf(sel_l[j] - m) / den;
    }
  }
}

// ============================================================== routing metadata
// Three short passes over the R = T*k slots, never leaving the GPU:
//   1. per-block expert histogram (blocks of kSlotsPerBlock slots)
//   2. one workgroup: per-expert exclusive scan over blocks, counts,
//      offsets = exclusive scan over experts, n_dropped
//   3. per block: stable rank of each slot among the block's slots of the
//      same expert (wave ballots over the id bits, waves in slot order),
//      giving row_of and src_slot.
constexpr int kSlotsPerBlock = 1024;
constexpr int kMetaThreads = 256;

__global__ void __launch_bounds__(kMetaThreads) hist_kernel(const int32_t* __restrict__ idx, int R,
                                                            int E, int32_t* __restrict__ hist,
                                                            int32_t* __restrict__ src_slot,
                                                            int n_rows, int32_t* err_flag) {
  __shared__ int h[MOE_MAX_EXPERTS];
  for (int e = threadIdx.x; e < E; e += kMetaThreads) h[e] = 0;
  __syncthreads();
  const int s0 = blockIdx.x * kSlotsPerBlock;
  bool bad = false;
  for (int i = threadIdx.x; i < kSlotsPerBlock; i += kMetaThreads) {
    const int s = s0 + i;
    if (s < R) {
      const int e = idx[s];
      if (e >= 0 && e < E) atomicAdd(&h[e], 1);
      else bad = true;
    }
  }
  if (bad) atomicOr(err_flag, 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kMetaThreads) hist[(size_t)blockIdx.x * E + e] = h[e];
  // every row starts as a pad row; pass 3 fills the live ones
  for (int r = blockIdx.x * kMetaThreads + threadIdx.x; r < n_rows; r += gridDim.x * kMetaThreads)
    src_slot[r] = -1;
}

// Block-wide exclusive scan of one int per thread (blockDim.x == 1024).
__device__ int block_exclusive_scan_1024(int v, int* total) {
  __shared__ int wsum[16];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int n = __shfl_up(incl, o, 64);
    if (lane >= o) incl += n;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  if (w == 0) {
    int s = lane < 16 ? wsum[lane] : 0;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const int n = __shfl_up(s, o, 64);
      if (lane >= o) s += n;
    }
    if (lane < 16) wsum[lane] = s;   // inclusive over waves
  }
  __syncthreads();
  const int before = (w > 0 ? wsum[w - 1] : 0) + incl - v;
  *total = wsum[15];
  return before;
}

// G threads (a power of two, G <= 64, within one wave) share expert e: each
// sums a run of blocks with independent loads, the group scans those sums,
// and each thread then writes the exclusive per-block bases of its run.
__global__ void __launch_bounds__(1024) scan_kernel(int32_t* __restrict__ hist, int nblk, int E,
                                                    int capacity, int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ offsets,
                                                    int32_t* __restrict__ n_dropped) {
  int G = 1;
  while (G * 2 * E <= 1024 && G * 2 <= 64) G *= 2;
  const int e = threadIdx.x / G, g = threadIdx.x % G;
  const bool live = e < E;
  const int per = (nblk + G - 1) / G;
  const int b0 = min(nblk, g * per), b1 = min(nblk, b0 + per);
  constexpr int kBurst = 16;
  int part = 0;
  if (live) {
    for (int b = b0; b < b1; b += kBurst) {
      int v[kBurst];
#pragma unroll
      for (int i = 0; i < kBurst; ++i) v[i] = b + i < b1 ? hist[(size_t)(b + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < kBurst; ++i) part += v[i];
    }
  }
  // inclusive scan of the partial sums over the G lanes of this expert
  const int lane = threadIdx.x & 63;
  int incl = part;
  for (int o = 1; o < G; o <<= 1) {
    const int n = __shfl_up(incl, o, 64);
    if ((lane % G) >= o) incl += n;
  }
  const int total = __shfl(incl, (lane / G) * G + G - 1, 64);
  if (live) {
    int run = incl - part;
    for (int b = b0; b < b1; b += kBurst) {
      int v[kBurst];
#pragma unroll
      for (int i = 0; i < kBurst; ++i) v[i] = b + i < b1 ? hist[(size_t)(b + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < kBurst; ++i) {
        if (b + i < b1) hist[(size_t)(b + i) * E + e] = run;
        run += v[i];
      }
    }
    if (g == 0) counts[e] = total;
  }
  __syncthreads();
  // exclusive scan of counts over experts: one thread per expert
  const int ce = threadIdx.x < E ? counts[threadIdx.x] : 0;
  int tot;
  const int off = block_exclusive_scan_1024(ce, &tot);
  if (threadIdx.x < E) offsets[threadIdx.x] = off;
  if (threadIdx.x == 0) offsets[E] = tot;
  const int drop = (capacity > 0 && threadIdx.x < E && ce > capacity) ? ce - capacity : 0;
  int dtotal;
  __syncthreads();
  (void)block_exclusive_scan_1024(drop, &dtotal);
  if (threadIdx.x == 0) *n_dropped = dtotal;
}

__global__ void __launch_bounds__(kMetaThreads) rank_kernel(
    const int32_t* __restrict__ idx, int R, int E, int capacity, const int32_t* __restrict__ hist,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ row_of, int32_t* __restrict__ src_slot) {
  constexpr int kWaves = kMetaThreads / 64;
  constexpr int kPerWave = kSlotsPerBlock / kWaves;
  __shared__ int base[kWaves][MOE_MAX_EXPERTS];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < kWaves * E; i += kMetaThreads) base[i / E][i % E] = 0;
  __syncthreads();
  const int s_wave = blockIdx.x * kSlotsPerBlock + w * kPerWave;
  for (int c = 0; c < kPerWave; c += 64) {
    const int s = s_wave + c + lane;
    const int e = s < R ? idx[s] : -1;
    if (e >= 0 && e < E) atomicAdd(&base[w][e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kMetaThreads) {
    int b = offsets[e] + hist[(size_t)blockIdx.x * E + e];
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const int n = base[ww][e];
      base[ww][e] = b;
      b += n;
    }
  }
  __syncthreads();
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int c = 0; c < kPerWave; c += 64) {
    const int s = s_wave + c + lane;
    const int e = s < R ? idx[s] : -1;
    const bool ok = e >= 0 && e < E;
    uint64_t peers = __ballot(ok);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = ok && ((e >> b) & 1);
      const uint64_t m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    int pos = 0;
    if (ok) {
      const int rank = __popcll(peers & lt);
      pos = base[w][e] + rank;
      if (rank == 0) base[w][e] = pos + __popcll(peers);
    }
    if (s < R) {
      int row = -1;
      if (ok) {
        if (capacity > 0) {
          const int r = pos - offsets[e];
          row = r < capacity ? e * capacity + r : -1;
        } else {
          row = pos;
        }
      }
      row_of[s] = row;
      if (row >= 0) src_slot[row] = s;
    }
  }
}

// ============================================================== router backward
__global__ void __launch_bounds__(256) route_bwd_kernel(const int32_t* __restrict__ idx,
                                                        const float* __restrict__ w,
                                                        const float* __restrict__ dw, int T_, int E,
                                                        int k, float* __restrict__ dl) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (size_t)T_ * E) return;
  const size_t t = i / E;
  const int e = static_cast<int>(i % E);
  float s = 0.f;
  int jj = -1;
  for (int j = 0; j < k; ++j) {
    s = fmaf(w[t * k + j], dw[t * k + j], s);
    if (jj < 0 && idx[t * k + j] == e) jj = j;
  }
  dl[i] = jj >= 0 ? w[t * k + jj] * (dw[t * k + jj] - s) : 0.f;
}

// dW_r = x^T dlogits, in two deterministic passes: partial sums over chunks
// of kRbTok tokens, then a fixed-order reduction over chunks.
constexpr int kRbTok = 128;
constexpr int kRbEC = 8;
constexpr int kRbCols = 64;             // vector columns per workgroup (one per lane)
constexpr int kRbWaveTok = kRbTok / 4;  // tokens of the chunk per wave

// Workgroup (chunk, column block, expert group): lane = vector column, wave
// = a quarter of the chunk's tokens (summed in order, eight rows in flight);
// the four quarters are added in wave order through LDS.
template <typename T>
__global__ void __launch_bounds__(256) router_bwd_partial_kernel(const T* __restrict__ x,
                                                                 const float* __restrict__ dl,
                                                                 int T_, int d, int E,
                                                                 float* __restrict__ part) {
  constexpr int V = kVec<T>;
  __shared__ float sdl[kRbTok][kRbEC];
  __shared__ float red[3][V * kRbEC][kRbCols];
  const int chunk = blockIdx.x;
  const int e0 = blockIdx.z * kRbEC;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = blockIdx.y * kRbCols + lane;             // vector column
  const int t0 = chunk * kRbTok;
  for (int i = threadIdx.x; i < kRbTok * kRbEC; i += 256) {
    const int tt = i / kRbEC, ee = i % kRbEC;
    sdl[tt][ee] = (t0 + tt < T_ && e0 + ee < E) ? dl[(size_t)(t0 + tt) * E + e0 + ee] : 0.f;
  }
  __syncthreads();
  const bool col = c * V < d;
  float acc[V][kRbEC];
#pragma unroll
  for (int a = 0; a < V; ++a)
#pragma unroll
    for (int b = 0; b < kRbEC; ++b) acc[a][b] = 0.f;
  const int tw0 = wave * kRbWaveTok;                      // first token of this wave (in the chunk)
  const int tn = min(kRbWaveTok, T_ - t0 - tw0);
  constexpr int kU = 8;
  for (int t1 = 0; col && t1 < tn; t1 += kU) {
    V16 xr[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (t1 + u < tn) xr[u] = *reinterpret_cast<const V16*>(x + (size_t)(t0 + tw0 + t1 + u) * d + (size_t)c * V);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (t1 + u < tn) {
        float xv[V];
        unpack(xr[u], xv);
#pragma unroll
        for (int b = 0; b < kRbEC; ++b) {
          const float g = sdl[tw0 + t1 + u][b];
#pragma unroll
          for (int a = 0; a < V; ++a) acc[a][b] = fmaf(xv[a], g, acc[a][b]);
        }
      }
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int a = 0; a < V; ++a)
#pragma unroll
      for (int b = 0; b < kRbEC; ++b) red[wave - 1][a * kRbEC + b][lane] = acc[a][b];
  }
  __syncthreads();
  if (wave == 0 && col) {
#pragma unroll
    for (int a = 0; a < V; ++a)
#pragma unroll
      for (int b = 0; b < kRbEC; ++b) {
        const float s = ((acc[a][b] + red[0][a * kRbEC + b][lane]) + red[1][a * kRbEC + b][lane]) +
                        red[2][a * kRbEC + b][lane];
        if (e0 + b < E) part[((size_t)chunk * d + c * V + a) * E + e0 + b] = s;
      }
  }
}

// dw_r[i] = sum over chunks of part[chunk][i]: eight lanes per output, lane j
// summing chunks j, j+8, ... in order, then a fixed shuffle tree.
constexpr int kRbRed = 8;
template <typename T>
__global__ void __launch_bounds__(256) router_bwd_reduce_kernel(const float* __restrict__ part,
                                                                int nchunk, int d, int E,
                                                                T* __restrict__ dw_r) {
  const size_t g = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t i = g / kRbRed;
  const int j = static_cast<int>(g % kRbRed);
  const size_t stride = (size_t)d * E;
  const bool live = i < stride;
  float s = 0.f;
  constexpr int kU = 4;
  for (int c = j; live && c < nchunk; c += kRbRed * kU) {
    float v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) v[u] = c + kRbRed * u < nchunk ? part[(size_t)(c + kRbRed * u) * stride + i] : 0.f;
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (c + kRbRed * u < nchunk) s += v[u];
  }
#pragma unroll
  for (int o = 1; o < kRbRed; o <<= 1) s += __shfl_xor(s, o, 64);
  if (live && j == 0) Elem<T>::store(dw_r, i, s);
}

}  // namespace moe

// ============================================================== C ABI
using namespace moe;

extern "C" int moe_router_gemm(int dtype, const void* x, const void* w_r, int T, int d, int E,
                               float* logits, hipStream_t stream) {
  MOE_CHECK_ARG(valid_dtype(dtype) && T >= 0 && d > 0 && E > 0 && d % 8 == 0);
  MOE_CHECK_SUPPORTED(E <= MOE_MAX_EXPERTS);
  if (T == 0) return MOE_OK;
  MOE_CHECK_ARG(x && w_r && logits && aligned16(x));
  const int waves = (T + kRouterTok - 1) / kRouterTok;
  const int blocks = (waves + 3) / 4;
  const bool wide = E % kRouterEC == 0 && aligned16(w_r);
  // w_r in LDS when it fits in 64 KB with its padding (four workgroups per CU)
  const long lds_bytes = (long)(d / 8) * router_lds_group_bytes(E);
  if (dtype == MOE_BF16 && wide && lds_bytes <= 64 * 1024) {
    router_gemm_lds_kernel<<<blocks, 256, lds_bytes, stream>>>(
        static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w_r), T, d, E, logits);
    return launch_status();
  }
  if (dtype == MOE_BF16)
    router_gemm_kernel<uint16_t><<<blocks, 256, 0, stream>>>(
        static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w_r), T, d, E, wide, logits);
  else
    router_gemm_kernel<float><<<blocks, 256, 0, stream>>>(static_cast<const float*>(x),
                                                          static_cast<const float*>(w_r), T, d, E,
                                                          wide, logits);
  return launch_status();
}

template <int L, int P>
static void launch_route(const float* logits, int T, int E, int k, int32_t* idx, float* w,
                         hipStream_t stream) {
  const long threads = (long)T * L;
  const int blocks = static_cast<int>((threads + 255) / 256);
  route_kernel<L, P><<<blocks, 256, 0, stream>>>(logits, T, E, k, idx, w);
}

extern "C" int moe_route(const float* logits, int T, int E, int k, int32_t* topk_idx,
                         float* topk_w, hipStream_t stream) {
  MOE_CHECK_ARG(T >= 0 && E > 0 && k >= 1 && k <= E);
  MOE_CHECK_SUPPORTED(E <= MOE_MAX_EXPERTS && k <= MOE_MAX_TOPK);
  if (T == 0) return MOE_OK;
  MOE_CHECK_ARG(logits && topk_idx && topk_w);
  if (E <= 1) launch_route<1, 1>(logits, T, E, k, topk_idx, topk_w, stream);
  else if (E <= 2) launch_route<2, 1>(logits, T, E, k, topk_idx, topk_w, stream);
  else if (E <= 4) launch_route<4, 1>(logits, T, E, k, topk_idx, topk_w, stream);
  else if (E <= 8) launch_route<8, 1>(logits, T, E, k, topk_idx, topk_w, stream);
  else if (E <= 16) launch_route<16, 1>(logits, T, E, k, topk_idx, topk_w, stream);
  else if (E <= 32) launch_route<32, 1>(logits, T, E, k, topk_idx, topk_w, stream);
  else if (E <= 64) launch_route<64, 1>(logits, T, E, k, topk_idx, topk_w, stream);
  else if (E <= 128) launch_route<64, 2>(logits, T, E, k, topk_idx, topk_w, stream);
  else if (E <= 256) launch_route<64, 4>(logits, T, E, k, topk_idx, topk_w, stream);
  else if (E <= 512) launch_route<64, 8>(logits, T, E, k, topk_idx, topk_w, stream);
  else launch_route<64, 16>(logits, T, E, k, topk_idx, topk_w, stream);
  return launch_status();
}

extern "C" size_t moe_offsets_workspace_bytes(int T, int k, int E) {
  if (T < 0 || k < 1 || E < 1) return 0;
  const long R = (long)T * k;
  const long nblk = (R + kSlotsPerBlock - 1) / kSlotsPerBlock;
  return static_cast<size_t>((nblk > 0 ? nblk : 1) * E * sizeof(int32_t));
}

extern "C" int moe_offsets(const int32_t* topk_idx, int T, int k, int E, int capacity,
                           int32_t* counts, int32_t* offsets, int32_t* row_of, int32_t* src_slot,
                           int32_t* n_dropped, int32_t* err_flag, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
  MOE_CHECK_ARG(counts && offsets && n_dropped && err_flag && T >= 0 && E > 0 && k >= 1 &&
                k <= E && capacity >= 0);
  MOE_CHECK_SUPPORTED(E <= MOE_MAX_EXPERTS && k <= MOE_MAX_TOPK);
  const long R = (long)T * k;
  MOE_CHECK_SUPPORTED(R < (1L << 31) && (long)E * capacity < (1L << 31));
  MOE_CHECK_ARG(R == 0 || (topk_idx && row_of));
  const long n_rows = capacity > 0 ? (long)E * capacity : R;
  MOE_CHECK_ARG(n_rows == 0 || src_slot);
  if (!ws || ws_bytes < moe_offsets_workspace_bytes(T, k, E)) return MOE_ERR_WORKSPACE;
  const int nblk = static_cast<int>(R > 0 ? (R + kSlotsPerBlock - 1) / kSlotsPerBlock : 1);
  int32_t* hist = static_cast<int32_t*>(ws);
  hist_kernel<<<nblk, kMetaThreads, 0, stream>>>(topk_idx, static_cast<int>(R), E, hist, src_slot,
                                                 static_cast<int>(n_rows), err_flag);
  if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
  scan_kernel<<<1, 1024, 0, stream>>>(hist, nblk, E, capacity, counts, offsets, n_dropped);
  if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
  rank_kernel<<<nblk, kMetaThreads, 0, stream>>>(topk_idx, static_cast<int>(R), E, capacity, hist,
                                                 offsets, row_of, src_slot);
  return launch_status();
}

extern "C" int moe_route_bwd(const int32_t* topk_idx, const float* topk_w, const float* dtopk_w,
                             int T, int E, int k, float* dlogits, hipStream_t stream) {
  MOE_CHECK_ARG(T >= 0 && E > 0 && k >= 1 && k <= E);
  MOE_CHECK_SUPPORTED(E <= MOE_MAX_EXPERTS && k <= MOE_MAX_TOPK);
  const size_t n = (size_t)T * E;
  if (n == 0) return MOE_OK;
  MOE_CHECK_ARG(topk_idx && topk_w && dtopk_w && dlogits);
  route_bwd_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, stream>>>(
      topk_idx, topk_w, dtopk_w, T, E, k, dlogits);
  return launch_status();
}

extern "C" size_t moe_router_bwd_workspace_bytes(int T, int d, int E) {
  if (T < 0 || d <= 0 || E <= 0) return 0;
  const size_t nchunk = (size_t)((T + kRbTok - 1) / kRbTok);
  return (nchunk > 0 ? nchunk : 1) * (size_t)d * E * sizeof(float);
}

extern "C" int moe_router_gemm_bwd(int dtype, const void* x, const float* dlogits, int T, int d,
                                   int E, void* dw_r, void* ws, size_t ws_bytes,
                                   hipStream_t stream) {
  MOE_CHECK_ARG(valid_dtype(dtype) && dw_r && T >= 0 && d > 0 && E > 0 && d % 8 == 0);
  MOE_CHECK_ARG(T == 0 || (x && dlogits && aligned16(x)));
  MOE_CHECK_SUPPORTED(E <= MOE_MAX_EXPERTS);
  if (!ws || ws_bytes < moe_router_bwd_workspace_bytes(T, d, E)) return MOE_ERR_WORKSPACE;
  const int nchunk = (T + kRbTok - 1) / kRbTok;
  float* part = static_cast<float*>(ws);
  const int V = dtype == MOE_BF16 ? 8 : 4;
  if (nchunk > 0) {
    dim3 grid(nchunk, (d / V + kRbCols - 1) / kRbCols, (E + kRbEC - 1) / kRbEC);
    if (dtype == MOE_BF16)
      router_bwd_partial_kernel<uint16_t><<<grid, 256, 0, stream>>>(
          static_cast<const uint16_t*>(x), dlogits, T, d, E, part);
    else
      router_bwd_partial_kernel<float><<<grid, 256, 0, stream>>>(static_cast<const float*>(x),
                                                                 dlogits, T, d, E, part);
    if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
  }
  const int nred = nchunk;   // T == 0: the reduction writes zeros
  const unsigned blocks = static_cast<unsigned>(((size_t)d * E * kRbRed + 255) / 256);
  if (dtype == MOE_BF16)
    router_bwd_reduce_kernel<uint16_t><<<blocks, 256, 0, stream>>>(part, nred, d, E,
                                                                   static_cast<uint16_t*>(dw_r));
  else
    router_bwd_reduce_kernel<float><<<blocks, 256, 0, stream>>>(part, nred, d, E,
                                                                static_cast<float*>(dw_r));
  return launch_status();
}
