// Router GEMM, top-k gate, GPU-resident routing metadata, and the router's
// backward (gfx950). See include/moe.h for the contract of each entry point.
#include "common.h"

#include <algorithm>
#include <mutex>

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
      // rows past T read row T-1 (a token's row feeds only its own logits,
      // which are not stored); a per-row branch would serialise the loads
      float xv[kRouterTok][V];
#pragma unroll
      for (int a = 0; a < kRouterTok; ++a) {
        V16 v = *reinterpret_cast<const V16*>(x + (size_t)min(t0 + a, T_ - 1) * d + (size_t)c * V);
        unpack(v, xv[a]);
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
          V16 v = *reinterpret_cast<const V16*>(x + (size_t)min(t0 + a, T_ - 1) * d + (size_t)c * V);
          unpack(v, xv[a]);
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

// The bf16 product on the matrix cores (E <= 16, E % 8 == 0, d % 256 == 0,
// d * E * 2 bytes of w_r fit in 64 KB): v_mfma_f32_16x16x32_bf16 with the
// tokens as rows (A: lane (r, g) holds x[t0 + r][k(s, g) .. + 7]) and the
// experts as columns (B: lane (r, g) holds w_r[k(s, g) .. + 7][r]). K step s
// takes the k order k(s, g) = 64 (s / 2) + 16 g + 8 (s % 2) (any order of the
// sum is the same product): each load instruction then touches whole
// 128-byte lines of its 16 rows (the four lanes of a row 32 bytes apart, the
// next step filling the gaps), which streams at about 5.4 TB/s where the
// plain order's 64-byte halves of 16 rows stay near 4.2.
//
// The product only streams x, so its rate is the number of x bytes in flight
// per CU. A workgroup of 16 waves takes 16 / SPLIT blocks of 16 tokens; the
// SPLIT waves of one block split d into chunks of kRmCh K steps dealt round
// robin (wave q takes chunks q, q + SPLIT, ...), issue the loads of all their
// chunks (NQ <= 2 of them: SPLIT is 4 up to d = 2048 and 8 above) before w_r
// is staged, and add their partial sums through LDS in the fixed order
// q = 0, 1, ..., SPLIT - 1 (the result does not depend on timing). w_r is staged once per workgroup in LDS in fragment
// order (the 64 lanes of one K step read one contiguous 1 KB). Columns r >= E
// read column E-1, rows past T read row T-1 and chunk indices past d re-read
// the last chunk: such an A row, B column or chunk feeds only an output that
// is not stored or a sum that skips it.
constexpr int kRmCh = 8;     // K steps (of 32) per chunk (even): 8 KB of x per wave per chunk
constexpr int kRmMaxLds = 64 * 1024;

static bool router_mfma_shape(int d, int E) {
  return E <= 16 && E % 8 == 0 && d % (32 * kRmCh) == 0 && (long)d * E * 2 <= kRmMaxLds;
}

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 rbf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float rf32x4_t;

// NQ: chunks per wave, ceil(d / (32 kRmCh) / SPLIT)
template <int NQ, int SPLIT>
__global__ void __launch_bounds__(1024) router_gemm_mfma_kernel(const uint16_t* __restrict__ x,
                                                                const uint16_t* __restrict__ w_r, int T_,
                                                                int d, int E, float* __restrict__ logits) {
  extern __shared__ __attribute__((aligned(16))) uint16_t wfrag[];   // [d/32][4][E][8]
  constexpr int BPW = 16 / SPLIT;                                     // blocks per workgroup
  __shared__ rf32x4_t part[16 * 64];                                  // [d part][block slot][lane]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, r = lane & 15;
  const int b = wave % BPW, q = wave / BPW;       // block slot, d part
  const int nblk = (T_ + 15) / 16;
  const int nch = d / (32 * kRmCh);
  rbf16x8_t a[NQ][kRmCh];
  auto load = [&](int blk) {
    const uint16_t* xr = x + (size_t)min(blk * 16 + r, T_ - 1) * d + g * 16;
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const int c = min(q + SPLIT * j, nch - 1);
#pragma unroll
      for (int s = 0; s < kRmCh; ++s)
        a[j][s] = *reinterpret_cast<const rbf16x8_t*>(xr + c * kRmCh * 32 + (s >> 1) * 64 + (s & 1) * 8);
    }
  };
  int base = blockIdx.x * BPW;
  load(base + b);
  // stage w_r: 16-byte pieces (8 experts of one row k) to fragment order,
  // two loads per thread in flight before their LDS writes (one round when
  // d * E <= 16384). A thread past the last piece re-reads a distinct real
  // piece (index mod pieces) rather than all of them one line.
  const int pieces = d * E / 8;
  for (int p0 = 0; p0 < pieces; p0 += 2048) {
    V16 v[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int p = p0 + j * 1024 + threadIdx.x;
      v[j] = reinterpret_cast<const V16*>(w_r)[p < pieces ? p : p % pieces];
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int p = p0 + j * 1024 + threadIdx.x;
      if (p >= pieces) break;
      // row k of w_r belongs to step s = 2 (k / 64) + (k / 8) % 2, lane group
      // g = (k % 64) / 16, element k % 8 of the fragment
      const int k = p * 8 / E, n0 = p * 8 % E;
      const int kk = k >> 3, st = (kk >> 3) * 2 + (kk & 1), gg = (kk >> 1) & 3;
      uint16_t* dst = wfrag + ((st * 4 + gg) * E + n0) * 8 + (k & 7);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dst[(2 * i) * 8] = static_cast<uint16_t>(v[j].w[i] & 0xffffu);
        dst[(2 * i + 1) * 8] = static_cast<uint16_t>(v[j].w[i] >> 16);
      }
    }
  }
  __syncthreads();
  const uint16_t* wl = wfrag + (g * E + min(r, E - 1)) * 8;
  // the loop condition is the same for every wave of the workgroup (barriers)
  for (; base < nblk; base += gridDim.x * BPW) {
    rf32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const int c = q + SPLIT * j;
      if (c < nch) {   // wave-uniform; no load sits under it
#pragma unroll
        for (int s = 0; s < kRmCh; ++s) {
          const rbf16x8_t bw = *reinterpret_cast<const rbf16x8_t*>(wl + (c * kRmCh + s) * 32 * E);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j][s], bw, acc, 0, 0, 0);
        }
      }
    }
    part[(q * BPW + b) * 64 + lane] = acc;
    // the next blocks' loads fly while the partials are added (only when this
    // workgroup has a next iteration: the condition is the same for all its
    // waves)
    if (base + (int)gridDim.x * BPW < nblk) load(base + (int)gridDim.x * BPW + b);
    __syncthreads();
    if (q == 0) {
      rf32x4_t sum = part[b * 64 + lane];
#pragma unroll
      for (int p = 1; p < SPLIT; ++p) {
        const rf32x4_t v = part[(p * BPW + b) * 64 + lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) sum[i] += v[i];
      }
      // lane (r, g) holds tokens 4g .. 4g+3 of the block, expert r
      if (r < E) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = (base + b) * 16 + 4 * g + i;
          if (t < T_) logits[(size_t)t * E + r] = sum[i];
        }
      }
    }
    __syncthreads();
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
// Short passes over the R = T*k slots, never leaving the GPU:
//   1. per-block expert histogram (blocks of kSlotsPerBlock slots)
//   2. counts, offsets (exclusive scan over experts), n_dropped and each
//      block's per-expert bases (sums over earlier blocks): inside pass 3
//      for small histograms, else one workgroup of its own
//   3. per block: stable rank of each slot among the block's slots of the
//      same expert, giving row_of and src_slot.
constexpr int kSlotsPerBlock = 1024;
constexpr int kMetaThreads = 256;
// Largest histogram (blocks x experts) every rank block sums itself: 64 KB of
// reads per block; larger ones go through scan_kernel first.
constexpr long kLocalScanMax = 16384;

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

// Pass 2 for large histograms (nblk * E above kLocalScanMax): one
// workgroup. G threads (a power of two, G <= 64, within one wave) share
// expert e: each sums a run of blocks with independent loads, the group
// scans those sums, and each thread then writes the exclusive per-block
// bases of its run over the histogram; then counts, offsets, n_dropped.
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

// Exclusive scan over the workgroup (kMetaThreads threads) of one int per
// thread; *total gets the sum.
__device__ int block_exclusive_scan(int v, int* total) {
  constexpr int kWaves = kMetaThreads / 64;
  __shared__ int wsum[kWaves];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int n = __shfl_up(incl, o, 64);
    if (lane >= o) incl += n;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int before = incl - v, all = 0;
#pragma unroll
  for (int j = 0; j < kWaves; ++j) {
    if (j < w) before += wsum[j];
    all += wsum[j];
  }
  __syncthreads();   // wsum may be reused by the next call
  *total = all;
  return before;
}

// Pass 3, with pass 2 folded in for small histograms (local_scan: nblk * E
// at most kLocalScanMax). Then every block sums the histogram's columns
// itself: over all blocks (the experts' counts, hence offsets and drops,
// the same in every block) and over the blocks before it (its own bases);
// block 0 writes counts, offsets and n_dropped. Otherwise scan_kernel has
// left each block's bases in the histogram and the offsets in `offsets`.
// Then the stable rank of each of the block's slots among its slots of the
// same expert (wave ballots over the id bits, waves in slot order) gives
// row_of and src_slot.
__global__ void __launch_bounds__(kMetaThreads) rank_kernel(
    const int32_t* __restrict__ idx, int R, int E, int capacity, const int32_t* __restrict__ hist, int nblk,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ n_dropped,
    int32_t* __restrict__ row_of, int32_t* __restrict__ src_slot, bool local_scan) {
  constexpr int kWaves = kMetaThreads / 64;
  constexpr int kPerWave = kSlotsPerBlock / kWaves;
  constexpr int kBurst = 16;
  __shared__ int tot_s[MOE_MAX_EXPERTS], pre_s[MOE_MAX_EXPERTS], off_s[MOE_MAX_EXPERTS];
  __shared__ int base[kWaves][MOE_MAX_EXPERTS];
  __shared__ int dropped_s;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int e = tid; e < E; e += kMetaThreads) {
    tot_s[e] = 0;
    pre_s[e] = 0;
  }
  for (int i = tid; i < kWaves * E; i += kMetaThreads) base[i / E][i % E] = 0;
  if (tid == 0) dropped_s = 0;
  __syncthreads();
  // column sums: P parts of the blocks per expert, bursts of independent
  // loads (indices clamped to the part, values past it masked)
  if (local_scan) {
    const int P = E >= kMetaThreads ? 1 : kMetaThreads / E;
    const int per = (nblk + P - 1) / P;
    for (int i = tid; i < E * P; i += kMetaThreads) {
      const int e = i % E, part = i / E;
      const int b0 = min(nblk, part * per), b1 = min(nblk, b0 + per);
      int tot = 0, pre = 0;
      for (int bb = b0; bb < b1; bb += kBurst) {
        int v[kBurst];
#pragma unroll
        for (int j = 0; j < kBurst; ++j) v[j] = hist[(size_t)min(bb + j, b1 - 1) * E + e];
#pragma unroll
        for (int j = 0; j < kBurst; ++j) {
          const int x = bb + j < b1 ? v[j] : 0;
          tot += x;
          pre += bb + j < (int)blockIdx.x ? x : 0;
        }
      }
      if (b0 < b1) {
        atomicAdd(&tot_s[e], tot);
        atomicAdd(&pre_s[e], pre);
      }
    }
  }
  // slots per wave and expert of this block
  const int s_wave = blockIdx.x * kSlotsPerBlock + w * kPerWave;
  for (int c = 0; c < kPerWave; c += 64) {
    const int s = s_wave + c + lane;
    const int e = s < R ? idx[s] : -1;
    if (e >= 0 && e < E) atomicAdd(&base[w][e], 1);
  }
  __syncthreads();
  // offsets: exclusive scan of the counts over experts (a run of consecutive
  // experts per thread); drops past the capacity
  if (!local_scan) {
    for (int e = tid; e < E; e += kMetaThreads) {
      off_s[e] = offsets[e];
      pre_s[e] = hist[(size_t)blockIdx.x * E + e];
    }
  } else {
    constexpr int kMaxRun = (MOE_MAX_EXPERTS + kMetaThreads - 1) / kMetaThreads;
    const int run = (E + kMetaThreads - 1) / kMetaThreads;
    const int e0 = tid * run;
    int sum = 0, drop = 0;
#pragma unroll
    for (int j = 0; j < kMaxRun; ++j) {
      const int e = e0 + j;
      if (j < run && e < E) {
        const int c = tot_s[e];
        sum += c;
        drop += capacity > 0 && c > capacity ? c - capacity : 0;
      }
    }
    int total;
    int before = block_exclusive_scan(sum, &total);
#pragma unroll
    for (int j = 0; j < kMaxRun; ++j) {
      const int e = e0 + j;
      if (j < run && e < E) {
        off_s[e] = before;
        before += tot_s[e];
      }
    }
    if (drop) atomicAdd(&dropped_s, drop);
    if (blockIdx.x == 0 && tid == 0) offsets[E] = total;
  }
  __syncthreads();
  if (local_scan && blockIdx.x == 0) {
    for (int e = tid; e < E; e += kMetaThreads) {
      counts[e] = tot_s[e];
      offsets[e] = off_s[e];
    }
    if (tid == 0) *n_dropped = dropped_s;
  }
  for (int e = tid; e < E; e += kMetaThreads) {
    int b = off_s[e] + pre_s[e];
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
          const int r = pos - off_s[e];
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

// The bf16 adjoint on the matrix cores (E <= 16, E % 4 == 0, d % 256 == 0): per
// workgroup a chunk of kRmTok tokens and 256 columns of x, part[chunk][i][e]
// = sum over the chunk of x[t][i] dl[t][e] as v_mfma_f32_16x16x32_bf16 with
// the experts as rows (A = dl^T) and the columns of x as columns (B = x, the
// contraction over tokens). dl is binary32; each value is carried as two
// bf16 terms, hi = bf16(dl) and lo = bf16(dl - hi) (dl - hi is exact), two
// MFMAs per fragment, so the products keep about 16 significant bits of dl
// against the 8 of one bf16 term. x tiles of 32 tokens x 256 columns move
// global -> registers (two K steps ahead) -> LDS (two buffers, 16-byte chunks
// XOR-swizzled by row) and are read down their columns with
// ds_read_b64_tr_b16. Tokens past T carry zero rows of x and zero dl.
constexpr int kRmTok = 256;               // tokens per chunk: eight K steps of 32
constexpr int kRmCols = 256;              // columns of x per workgroup (64 per wave)
constexpr int kRmDlLd = kRmTok + 8;       // dl^T row stride in LDS (bf16)

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short rs4_t;
MOE_DEV rbf16x8_t lds_tr8(const uint16_t* p0, const uint16_t* p1) {
  const rs4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) rs4_t*)p0);
  const rs4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) rs4_t*)p1);
  typedef __attribute__((__vector_size__(8 * sizeof(short)))) short s8_t;
  const s8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(rbf16x8_t, v);
}
// 16-byte chunk position of chunk c in LDS row k of an x tile: the 16 rows
// one transposed read touches (k = 8 tg + tj, tg, tj < 4) land on 16
// different chunk pairs
MOE_DEV int rm_chunk(int k, int c) { return c ^ (((k & 3) | ((k >> 3) & 3) << 2) << 1); }

__global__ void __launch_bounds__(256) router_bwd_mfma_kernel(const uint16_t* __restrict__ x,
                                                              const float* __restrict__ dl, int T_, int d,
                                                              int E, float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][32 * kRmCols];
  __shared__ __attribute__((aligned(16))) uint16_t dlh[16 * kRmDlLd];
  __shared__ __attribute__((aligned(16))) uint16_t dll[16 * kRmDlLd];
  const int chunk = blockIdx.x, c0 = blockIdx.y * kRmCols;
  const int t0 = chunk * kRmTok;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // x tile loads: thread tid moves 16-byte chunks tid + 256 j (j < 4) of the
  // 32 x 32-chunk tile: row (tid >> 5) + 8 j, chunk tid & 31
  const int lrow = tid >> 5, lch = tid & 31;
  auto load = [&](int ks, V16 (&v)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = min(t0 + ks * 32 + lrow + 8 * j, T_ - 1);
      v[j] = *reinterpret_cast<const V16*>(x + (size_t)t * d + c0 + lch * 8);
    }
  };
  auto store = [&](int ks, const V16 (&v)[4], uint16_t* buf) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = lrow + 8 * j;
      const bool ok = t0 + ks * 32 + k < T_;
      V16 o;   // selected word by word (a select of whole vectors went through scratch memory)
#pragma unroll
      for (int i = 0; i < 4; ++i) o.w[i] = ok ? v[j].w[i] : 0u;
      *reinterpret_cast<V16*>(buf + k * kRmCols + rm_chunk(k, lch) * 8) = o;
    }
  };
  V16 ra[4], rb[4];
  load(0, ra);
  load(1, rb);
  // dl^T of the chunk as hi/lo bf16 pairs: the chunk's kRmTok x E binary32
  // values are contiguous; four 16-byte loads per thread (E % 4 == 0, so a
  // piece never straddles two tokens), issued together, tokens past T zero.
  // Rows e >= E of dl^T stay unwritten: an A row feeds only its own output
  // row, which is not stored.
  {
    const float4* src = reinterpret_cast<const float4*>(dl + (size_t)t0 * E);
    const int np = kRmTok * E / 4, nvalid = (min(kRmTok, T_ - t0) * E) / 4;
    float4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = src[min(tid + 256 * j, nvalid - 1)];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int q = tid + 256 * j;
      if (q < np) {
        const int t = q * 4 / E, e0 = q * 4 % E;
        const float f[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float fv = q < nvalid ? f[i] : 0.f;
          const uint16_t h = f32_to_bf16(fv);
          dlh[(e0 + i) * kRmDlLd + t] = h;
          dll[(e0 + i) * kRmDlLd + t] = f32_to_bf16(fv - bf16_to_f32(h));
        }
      }
    }
  }
  store(0, ra, xs[0]);
  load(2, ra);
  __syncthreads();

  const int g = lane >> 4, r = lane & 15;
  const int tj = (lane & 15) >> 2, tq = lane & 3;
  rf32x4_t acc[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) acc[n] = rf32x4_t{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int ks, const uint16_t* buf) {
    const rbf16x8_t ah = *reinterpret_cast<const rbf16x8_t*>(dlh + r * kRmDlLd + ks * 32 + 8 * g);
    const rbf16x8_t al = *reinterpret_cast<const rbf16x8_t*>(dll + r * kRmDlLd + ks * 32 + 8 * g);
    const int k0 = 8 * g + tj, k1 = k0 + 4;
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int col = wave * 64 + n * 16 + 4 * tq;
      const rbf16x8_t b = lds_tr8(buf + k0 * kRmCols + rm_chunk(k0, col >> 3) * 8 + (col & 7),
                                  buf + k1 * kRmCols + rm_chunk(k1, col >> 3) * 8 + (col & 7));
      acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, b, acc[n], 0, 0, 0);
      acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, b, acc[n], 0, 0, 0);
    }
  };
  // eight K steps, two buffers; step ks + 1 waits in registers and goes to
  // LDS after step ks, whose barrier also ends every read of that buffer's
  // previous contents (step ks - 1)
#pragma unroll
  for (int ks = 0; ks < kRmTok / 32; ++ks) {
    compute(ks, xs[ks & 1]);
    if (ks + 1 < kRmTok / 32) {
      if (ks & 1) {
        store(ks + 1, ra, xs[(ks + 1) & 1]);
        if (ks + 3 < kRmTok / 32) load(ks + 3, ra);
      } else {
        store(ks + 1, rb, xs[(ks + 1) & 1]);
        if (ks + 3 < kRmTok / 32) load(ks + 3, rb);
      }
    }
    __syncthreads();
  }
  // lane (r, g) holds experts 4g .. 4g+3 of column r of each 16-column tile
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int col = c0 + wave * 64 + n * 16 + r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * g + i;
      if (e < E) part[((size_t)chunk * d + col) * E + e] = acc[n][i];
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
  const bool wide = E % kRouterEC == 0 && aligned16(w_r);
  if (dtype == MOE_BF16 && wide && router_mfma_shape(d, E)) {
    // 16 / split blocks of 16 tokens per workgroup of 16 waves, at most 256
    // workgroups (one per CU); dynamic LDS holds w_r
    const long nblk = (T + 15) / 16;
    const int nch = d / (32 * kRmCh);                 // 1..16 under the 64 KB w_r limit
    const int split = nch <= 8 ? 4 : 8;
    const int nq = (nch + split - 1) / split;         // 1 or 2
    const int bpw = 16 / split;
    const int blocks = static_cast<int>(std::min<long>(256, (nblk + bpw - 1) / bpw));
    const size_t lds = (size_t)d * E * 2;
    const auto* xp = static_cast<const uint16_t*>(x);
    const auto* wp = static_cast<const uint16_t*>(w_r);
    if (split == 4 && nq == 1) router_gemm_mfma_kernel<1, 4><<<blocks, 1024, lds, stream>>>(xp, wp, T, d, E, logits);
    else if (split == 4) router_gemm_mfma_kernel<2, 4><<<blocks, 1024, lds, stream>>>(xp, wp, T, d, E, logits);
    else router_gemm_mfma_kernel<2, 8><<<blocks, 1024, lds, stream>>>(xp, wp, T, d, E, logits);
    return launch_status();
  }
  const int waves = (T + kRouterTok - 1) / kRouterTok;
  const int blocks = (waves + 3) / 4;
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

// ---------------------------------------------------------------- no-allocation variant
// moe_offsets_noalloc keeps the per-block histogram in this file-scope device
// array instead of a caller workspace. Every GPU the library runs on holds
// its own copy until the process ends. In host code the name `scratch` is
// only a stand-in: the device address of each GPU's copy comes from
// hipGetSymbolAddress, looked up once per device with that device current
// and kept in scratch_addr.
constexpr size_t kOffsetsScratchBytes = MOE_OFFSETS_NOALLOC_MAX_BYTES;
static __device__ __align__(256) int32_t scratch[kOffsetsScratchBytes / sizeof(int32_t)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_addr[kMaxDevices] = {};

// Device address of the current device's scratch array, or nullptr when it
// cannot be resolved.
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    scratch_addr[dev] = p;
  }
  return scratch_addr[dev];
}
}  // namespace

extern "C" int moe_offsets_noalloc(const int32_t* topk_idx, int T, int k, int E, int capacity,
                                   int32_t* counts, int32_t* offsets, int32_t* row_of,
                                   int32_t* src_slot, int32_t* n_dropped, int32_t* err_flag,
                                   hipStream_t stream) {
  // the same argument checks as moe_offsets, before the scratch is looked up
  MOE_CHECK_ARG(counts && offsets && n_dropped && err_flag && T >= 0 && E > 0 && k >= 1 &&
                k <= E && capacity >= 0);
  MOE_CHECK_SUPPORTED(E <= MOE_MAX_EXPERTS && k <= MOE_MAX_TOPK);
  const long R = (long)T * k;
  MOE_CHECK_SUPPORTED(R < (1L << 31) && (long)E * capacity < (1L << 31));
  const size_t need = moe_offsets_workspace_bytes(T, k, E);
  MOE_CHECK_SUPPORTED(need <= kOffsetsScratchBytes);   // beyond the array: not this entry point
  void* ws = device_scratch();
  if (ws == nullptr) return MOE_ERR_HIP;
  // every histogram entry the call reads is written by the call first: nothing to clear
  return moe_offsets(topk_idx, T, k, E, capacity, counts, offsets, row_of, src_slot, n_dropped,
                     err_flag, ws, kOffsetsScratchBytes, stream);
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
  const bool local_scan = static_cast<long>(nblk) * E <= kLocalScanMax;
  if (!local_scan) {
    scan_kernel<<<1, 1024, 0, stream>>>(hist, nblk, E, capacity, counts, offsets, n_dropped);
    if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
  }
  rank_kernel<<<nblk, kMetaThreads, 0, stream>>>(topk_idx, static_cast<int>(R), E, capacity, hist, nblk,
                                                 counts, offsets, n_dropped, row_of, src_slot, local_scan);
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
  float* part = static_cast<float*>(ws);
  if (dtype == MOE_BF16 && E <= 16 && E % 4 == 0 && d % kRmCols == 0 && aligned16(x) && aligned16(dlogits)) {
    const int nch = (T + kRmTok - 1) / kRmTok;   // fewer chunks than the workspace is sized for
    if (nch > 0) {
      router_bwd_mfma_kernel<<<dim3(nch, d / kRmCols), 256, 0, stream>>>(static_cast<const uint16_t*>(x), dlogits,
                                                                        T, d, E, part);
      if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
    }
    const unsigned blocks = static_cast<unsigned>(((size_t)d * E * kRbRed + 255) / 256);
    router_bwd_reduce_kernel<uint16_t><<<blocks, 256, 0, stream>>>(part, nch, d, E, static_cast<uint16_t*>(dw_r));
    return launch_status();
  }
  const int nchunk = (T + kRbTok - 1) / kRbTok;
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
