// Row movement between token order and expert order (gfx950): permute,
// weighted combine, and their adjoints. HBM-bound: one wave per token row,
// 16-byte loads and stores, every token row read once and every routed row
// written once. See include/moe.h for the contract of each entry point.
#include "common.h"

namespace moe {

constexpr int kRowThreads = 256;   // 4 waves = 4 tokens per workgroup
// 16-byte pieces per lane taken together: a wave moves 4 KB of one row (a
// whole d = 2048 bf16 row) before it turns to the next row
constexpr int kRowUnroll = 4;

// Every load below is unconditional: a piece index past the row is clamped to
// the row's last piece and a missing row is replaced by a valid one, the
// result then discarded or zeroed by a select. A load under a per-lane or
// per-row branch is followed by a wait for it at the branch's end, which
// leaves one load in flight per wave; these kernels move rows and live on
// the loads they keep in flight.

// The token's row ids (k <= 16 <= 64): lane j < k holds slot j's row, -1 for
// a slot past k or an id outside [0, n_rows) (skipped, never dereferenced).
// One load per lane; slot j's row is then slot_row(rid, j), wave-uniform.
MOE_DEV int load_row_ids(const int32_t* row_of, size_t t, int k, int n_rows, int lane) {
  const int r = row_of[t * k + min(lane, k - 1)];
  return lane < k && r >= 0 && r < n_rows ? r : -1;
}
MOE_DEV int slot_row(int rid, int j) { return __builtin_amdgcn_readlane(rid, j); }
MOE_DEV float slot_val(float v, int j) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), j)); }

// Holds a loaded vector in registers from here on. Without it the compiler
// may move a load down to each of its conditional uses (a store per routed
// row, an FMA per valid slot) and reload it there, one wait per use.
MOE_DEV void pin(V16& v) { asm volatile("" : "+v"(v.w[0]), "+v"(v.w[1]), "+v"(v.w[2]), "+v"(v.w[3])); }

// x_perm[row_of[t, j]] = x[t]
template <typename T>
__global__ void __launch_bounds__(kRowThreads) permute_kernel(const T* __restrict__ x, int T_, int d,
                                                              int k, const int32_t* __restrict__ row_of,
                                                              int n_rows, T* __restrict__ x_perm) {
  constexpr int V = kVec<T>;
  const size_t t = ((size_t)blockIdx.x * kRowThreads + threadIdx.x) >> 6;
  const int lane = threadIdx.x & 63;
  if (t >= (size_t)T_) return;
  const int nvec = d / V;
  const V16* src = reinterpret_cast<const V16*>(x + t * d);
  // kRowUnroll 1 KB pieces of the row at once, then each destination row
  // written piece after piece; the first pieces are in flight before the row
  // ids are asked for
  V16 v[kRowUnroll];
  auto load = [&](int c0) {
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) v[u] = src[min(c0 + 64 * u, nvec - 1)];
  };
  load(lane);
  const int rid = load_row_ids(row_of, t, k, n_rows, lane);
  for (int c0 = lane;;) {
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) pin(v[u]);
    for (int j = 0; j < k; ++j) {
      const int r = slot_row(rid, j);
      if (r < 0) continue;
      V16* dst = reinterpret_cast<V16*>(x_perm + (size_t)r * d);
#pragma unroll
      for (int u = 0; u < kRowUnroll; ++u)
        if (c0 + 64 * u < nvec) dst[c0 + 64 * u] = v[u];
    }
    c0 += 64 * kRowUnroll;
    if (c0 - lane >= nvec) break;   // wave-uniform
    load(c0);
  }
}

// Zero the rows r with src_slot[r] == -1 (pad rows of the padded layout).
template <typename T>
__global__ void __launch_bounds__(kRowThreads) zero_pad_rows_kernel(const int32_t* __restrict__ src_slot,
                                                                    int n_rows, int d, T* __restrict__ buf) {
  constexpr int V = kVec<T>;
  const size_t r = ((size_t)blockIdx.x * kRowThreads + threadIdx.x) >> 6;
  const int lane = threadIdx.x & 63;
  if (r >= (size_t)n_rows || src_slot[r] != -1) return;
  V16 z;
#pragma unroll
  for (int i = 0; i < 4; ++i) z.w[i] = 0u;
  V16* dst = reinterpret_cast<V16*>(buf + r * d);
  for (int c = lane; c < d / V; c += 64) dst[c] = z;
}

// y[t] = y_add[t] + sum_j w[t, j] y_perm[row_of[t, j]]  (binary32, slot order;
// y_add optional). Source rows are read in groups of kRowGroup slots, all
// their pieces in flight together; a missing row reads the token's first
// valid row and adds nothing.
constexpr int kRowGroup = 4;
template <typename T>
__global__ void __launch_bounds__(kRowThreads) combine_kernel(const T* __restrict__ y_perm,
                                                              const int32_t* __restrict__ row_of,
                                                              const float* __restrict__ topk_w, int T_,
                                                              int k, int d, int n_rows,
                                                              const T* __restrict__ y_add,
                                                              T* __restrict__ y) {
  constexpr int V = kVec<T>;
  const size_t t = ((size_t)blockIdx.x * kRowThreads + threadIdx.x) >> 6;
  const int lane = threadIdx.x & 63;
  if (t >= (size_t)T_) return;
  const int rid = load_row_ids(row_of, t, k, n_rows, lane);
  const float wl = topk_w[t * k + min(lane, k - 1)];
  int first = -1;
  for (int j = k - 1; j >= 0; --j) first = slot_row(rid, j) >= 0 ? slot_row(rid, j) : first;
  const int nvec = d / V;
  for (int c0 = lane; c0 < nvec; c0 += 64 * kRowUnroll) {
    float acc[kRowUnroll][V];
    if (y_add) {
      V16 a[kRowUnroll];
#pragma unroll
      for (int u = 0; u < kRowUnroll; ++u) a[u] = reinterpret_cast<const V16*>(y_add + t * d)[min(c0 + 64 * u, nvec - 1)];
#pragma unroll
      for (int u = 0; u < kRowUnroll; ++u) unpack(a[u], acc[u]);
    } else {
#pragma unroll
      for (int u = 0; u < kRowUnroll; ++u)
#pragma unroll
        for (int i = 0; i < V; ++i) acc[u][i] = 0.f;
    }
    if (first >= 0) {
      for (int j0 = 0; j0 < k; j0 += kRowGroup) {
        V16 v[kRowGroup][kRowUnroll];
#pragma unroll
        for (int jj = 0; jj < kRowGroup; ++jj) {
          const int r = slot_row(rid, min(j0 + jj, 63));
          const V16* src = reinterpret_cast<const V16*>(y_perm + (size_t)(r >= 0 ? r : first) * d);
#pragma unroll
          for (int u = 0; u < kRowUnroll; ++u) v[jj][u] = src[min(c0 + 64 * u, nvec - 1)];
        }
#pragma unroll
        for (int jj = 0; jj < kRowGroup; ++jj)
#pragma unroll
          for (int u = 0; u < kRowUnroll; ++u) pin(v[jj][u]);
#pragma unroll
        for (int jj = 0; jj < kRowGroup; ++jj) {
          if (slot_row(rid, min(j0 + jj, 63)) < 0) continue;   // wave-uniform
          const float w = slot_val(wl, j0 + jj);
#pragma unroll
          for (int u = 0; u < kRowUnroll; ++u) {
            float f[V];
            unpack(v[jj][u], f);
#pragma unroll
            for (int i = 0; i < V; ++i) acc[u][i] = fmaf(w, f[i], acc[u][i]);
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u)
      if (c0 + 64 * u < nvec) reinterpret_cast<V16*>(y + t * d)[c0 + 64 * u] = pack(acc[u]);
  }
}

// dy_perm[row_of[t, j]] = w[t, j] dy[t];  dw[t, j] = <dy[t], y_perm[row_of[t, j]]>
// Slots in groups of kRowGroup: the token's dy pieces and the group's routed
// rows are in flight together; a missing row reads the token's first valid
// row, its product and store skipped.
template <typename T>
__global__ void __launch_bounds__(kRowThreads) combine_bwd_kernel(
    const T* __restrict__ dy, const T* __restrict__ y_perm, const float* __restrict__ topk_w,
    const int32_t* __restrict__ row_of, int T_, int k, int d, int n_rows, T* __restrict__ dy_perm,
    float* __restrict__ dtopk_w) {
  constexpr int V = kVec<T>;
  const size_t t = ((size_t)blockIdx.x * kRowThreads + threadIdx.x) >> 6;
  const int lane = threadIdx.x & 63;
  if (t >= (size_t)T_) return;
  const int rid = load_row_ids(row_of, t, k, n_rows, lane);
  const float wl = topk_w[t * k + min(lane, k - 1)];
  int first = -1;
  for (int j = k - 1; j >= 0; --j) first = slot_row(rid, j) >= 0 ? slot_row(rid, j) : first;
  const int nvec = d / V;
  const V16* g_row = reinterpret_cast<const V16*>(dy + t * d);
  float dotl = 0.f;   // lane j: slot j's dot product
  for (int j0 = 0; first >= 0 && j0 < k; j0 += kRowGroup) {
    float dot[kRowGroup] = {};
    int rr[kRowGroup];
#pragma unroll
    for (int jj = 0; jj < kRowGroup; ++jj) rr[jj] = slot_row(rid, min(j0 + jj, 63));
    for (int c0 = lane; c0 < nvec; c0 += 64 * kRowUnroll) {
      V16 gv[kRowUnroll], v[kRowGroup][kRowUnroll];
#pragma unroll
      for (int u = 0; u < kRowUnroll; ++u) gv[u] = g_row[min(c0 + 64 * u, nvec - 1)];
#pragma unroll
      for (int jj = 0; jj < kRowGroup; ++jj) {
        const V16* src = reinterpret_cast<const V16*>(y_perm + (size_t)(rr[jj] >= 0 ? rr[jj] : first) * d);
#pragma unroll
        for (int u = 0; u < kRowUnroll; ++u) v[jj][u] = src[min(c0 + 64 * u, nvec - 1)];
      }
#pragma unroll
      for (int u = 0; u < kRowUnroll; ++u) {
        pin(gv[u]);
#pragma unroll
        for (int jj = 0; jj < kRowGroup; ++jj) pin(v[jj][u]);
      }
#pragma unroll
      for (int jj = 0; jj < kRowGroup; ++jj) {
        if (rr[jj] < 0) continue;   // wave-uniform
        const float w = slot_val(wl, j0 + jj);
        V16* dst = reinterpret_cast<V16*>(dy_perm + (size_t)rr[jj] * d);
#pragma unroll
        for (int u = 0; u < kRowUnroll; ++u) {
          if (c0 + 64 * u >= nvec) continue;
          float g[V], f[V], o[V];
          unpack(gv[u], g);
          unpack(v[jj][u], f);
#pragma unroll
          for (int i = 0; i < V; ++i) {
            dot[jj] = fmaf(g[i], f[i], dot[jj]);
            o[i] = w * g[i];
          }
          dst[c0 + 64 * u] = pack(o);
        }
      }
    }
#pragma unroll
    for (int jj = 0; jj < kRowGroup; ++jj) {
      const float sdot = wave_sum(dot[jj]);
      if (lane == j0 + jj) dotl = sdot;
    }
  }
  if (lane < k) dtopk_w[t * k + lane] = rid >= 0 ? dotl : 0.f;
}

// The same adjoint in row order, for callers that have src_slot: wave r
// handles routed row r, s = src_slot[r], t = s / k:
//   dy_perm[r] = w[s] dy[t],  dtopk_w[s] = <dy[t], y_perm[r]>,
// and writes a zero row for a pad row (s == -1). y_perm is then read and
// dy_perm written in address order, while the dy rows (T x d, read k times)
// come mostly from cache: faster than the token-order form, whose k routed
// rows per token lie anywhere. The workgroups past the row grid give every
// slot without a row (dropped, or a bad expert id) dtopk_w = 0.
template <typename T>
__global__ void __launch_bounds__(kRowThreads) combine_bwd_rows_kernel(
    const T* __restrict__ dy, const T* __restrict__ y_perm, const float* __restrict__ topk_w,
    const int32_t* __restrict__ row_of, const int32_t* __restrict__ src_slot, int T_, int k, int d,
    int n_rows, int row_blocks, T* __restrict__ dy_perm, float* __restrict__ dtopk_w) {
  constexpr int V = kVec<T>;
  const size_t slots = (size_t)T_ * k;
  if ((int)blockIdx.x >= row_blocks) {
    const size_t s = (size_t)(blockIdx.x - row_blocks) * kRowThreads + threadIdx.x;
    if (s < slots) {
      const int r = row_of[s];
      if (r < 0 || r >= n_rows) dtopk_w[s] = 0.f;
    }
    return;
  }
  const size_t r = ((size_t)blockIdx.x * kRowThreads + threadIdx.x) >> 6;
  const int lane = threadIdx.x & 63;
  if (r >= (size_t)n_rows) return;
  const int nvec = d / V;
  V16* dst = reinterpret_cast<V16*>(dy_perm + r * d);
  const V16* y_row = reinterpret_cast<const V16*>(y_perm + r * d);
  // the routed row's first pieces do not depend on its slot: in flight
  // before the slot id arrives
  V16 yv[kRowUnroll];
#pragma unroll
  for (int u = 0; u < kRowUnroll; ++u) yv[u] = y_row[min(lane + 64 * u, nvec - 1)];
  const int s = __builtin_amdgcn_readfirstlane(src_slot[r]);
  if (s < 0 || (size_t)s >= slots) {
    V16 z;
#pragma unroll
    for (int i = 0; i < 4; ++i) z.w[i] = 0u;
    for (int c = lane; c < nvec; c += 64) dst[c] = z;
    return;
  }
  const float w = topk_w[s];
  const V16* g_row = reinterpret_cast<const V16*>(dy + (size_t)(s / k) * d);
  float dot = 0.f;
  for (int c0 = lane; c0 < nvec; c0 += 64 * kRowUnroll) {
    V16 gv[kRowUnroll];
    if (c0 != lane) {
#pragma unroll
      for (int u = 0; u < kRowUnroll; ++u) yv[u] = y_row[min(c0 + 64 * u, nvec - 1)];
    }
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) gv[u] = g_row[min(c0 + 64 * u, nvec - 1)];
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
      pin(gv[u]);
      pin(yv[u]);
    }
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
      if (c0 + 64 * u < nvec) {
        float g[V], f[V], o[V];
        unpack(gv[u], g);
        unpack(yv[u], f);
#pragma unroll
        for (int i = 0; i < V; ++i) {
          dot = fmaf(g[i], f[i], dot);
          o[i] = w * g[i];
        }
        dst[c0 + 64 * u] = pack(o);
      }
    }
  }
  dot = wave_sum(dot);
  if (lane == 0) dtopk_w[s] = dot;
}

// dx[t] = dx_add[t] + sum_j dx_perm[row_of[t, j]] (+ sum_e dlogits[t, e] w_r[:, e]);
// dx_add and the router term optional
template <typename T>
__global__ void __launch_bounds__(kRowThreads) permute_bwd_kernel(
    const T* __restrict__ dx_perm, const int32_t* __restrict__ row_of, int T_, int k, int d,
    int n_rows, const float* __restrict__ dlogits, const T* __restrict__ w_r, int E,
    const T* __restrict__ dx_add, T* __restrict__ dx) {
  constexpr int V = kVec<T>;
  const size_t t = ((size_t)blockIdx.x * kRowThreads + threadIdx.x) >> 6;
  const int lane = threadIdx.x & 63;
  if (t >= (size_t)T_) return;
  const int rid = load_row_ids(row_of, t, k, n_rows, lane);
  int first = -1;
  for (int j = k - 1; j >= 0; --j) first = slot_row(rid, j) >= 0 ? slot_row(rid, j) : first;
  const int nvec = d / V;
  const bool router = dlogits != nullptr;
  const bool wide = router && (E % V == 0);
  for (int c0 = lane; c0 < nvec; c0 += 64 * kRowUnroll) {
    float acc[kRowUnroll][V];
    if (dx_add) {
      V16 a[kRowUnroll];
#pragma unroll
      for (int u = 0; u < kRowUnroll; ++u) a[u] = reinterpret_cast<const V16*>(dx_add + t * d)[min(c0 + 64 * u, nvec - 1)];
#pragma unroll
      for (int u = 0; u < kRowUnroll; ++u) unpack(a[u], acc[u]);
    } else {
#pragma unroll
      for (int u = 0; u < kRowUnroll; ++u)
#pragma unroll
        for (int i = 0; i < V; ++i) acc[u][i] = 0.f;
    }
    // source rows in groups of kRowGroup slots, all their pieces in flight
    // together, added in slot order
    if (first >= 0) {
      for (int j0 = 0; j0 < k; j0 += kRowGroup) {
        V16 v[kRowGroup][kRowUnroll];
#pragma unroll
        for (int jj = 0; jj < kRowGroup; ++jj) {
          const int r = slot_row(rid, min(j0 + jj, 63));
          const V16* src = reinterpret_cast<const V16*>(dx_perm + (size_t)(r >= 0 ? r : first) * d);
#pragma unroll
          for (int u = 0; u < kRowUnroll; ++u) v[jj][u] = src[min(c0 + 64 * u, nvec - 1)];
        }
#pragma unroll
        for (int jj = 0; jj < kRowGroup; ++jj)
#pragma unroll
          for (int u = 0; u < kRowUnroll; ++u) pin(v[jj][u]);
#pragma unroll
        for (int jj = 0; jj < kRowGroup; ++jj) {
          if (slot_row(rid, min(j0 + jj, 63)) < 0) continue;   // wave-uniform
#pragma unroll
          for (int u = 0; u < kRowUnroll; ++u) {
            float f[V];
            unpack(v[jj][u], f);
#pragma unroll
            for (int i = 0; i < V; ++i) acc[u][i] += f[i];
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
      const int c = c0 + 64 * u;
      if (c >= nvec) continue;
      if (wide) {
        // w_r rows c*V .. c*V+V-1 are contiguous runs of E values
        for (int e0 = 0; e0 < E; e0 += V) {
          float g[V];
#pragma unroll
          for (int ee = 0; ee < V; ++ee) g[ee] = dlogits[t * E + e0 + ee];
#pragma unroll
          for (int i = 0; i < V; ++i) {
            float wv[V];
            unpack(*reinterpret_cast<const V16*>(w_r + (size_t)(c * V + i) * E + e0), wv);
#pragma unroll
            for (int ee = 0; ee < V; ++ee) acc[u][i] = fmaf(g[ee], wv[ee], acc[u][i]);
          }
        }
      } else if (router) {
        for (int e = 0; e < E; ++e) {
          const float g = dlogits[t * E + e];
#pragma unroll
          for (int i = 0; i < V; ++i) acc[u][i] = fmaf(g, Elem<T>::load(w_r, (size_t)(c * V + i) * E + e), acc[u][i]);
        }
      }
      reinterpret_cast<V16*>(dx + t * d)[c] = pack(acc[u]);
    }
  }
}

}  // namespace moe

// ============================================================== C ABI
using namespace moe;

namespace {

int row_grid(long rows) { return static_cast<int>((rows * 64 + kRowThreads - 1) / kRowThreads); }

int check_rows(int dtype, int T, int d, int k, int n_rows) {
  MOE_CHECK_ARG(valid_dtype(dtype) && T >= 0 && d > 0 && k >= 1 && n_rows >= 0);
  MOE_CHECK_ARG(d % 8 == 0);
  MOE_CHECK_SUPPORTED(k <= MOE_MAX_TOPK && (long)T * k < (1L << 31));
  return MOE_OK;
}

template <typename T>
int zero_pads(const int32_t* src_slot, int n_rows, int d, void* buf, hipStream_t stream) {
  if (n_rows == 0) return MOE_OK;
  zero_pad_rows_kernel<T><<<row_grid(n_rows), kRowThreads, 0, stream>>>(src_slot, n_rows, d,
                                                                         static_cast<T*>(buf));
  return launch_status();
}

}  // namespace

extern "C" int moe_permute(int dtype, const void* x, int T, int d, int k, const int32_t* row_of,
                           const int32_t* src_slot, int n_rows, void* x_perm, hipStream_t stream) {
  if (int st = check_rows(dtype, T, d, k, n_rows)) return st;
  MOE_CHECK_ARG(src_slot || (long)n_rows == (long)T * k);
  MOE_CHECK_ARG((T == 0 || (x && row_of && aligned16(x))) && (n_rows == 0 || (x_perm && aligned16(x_perm))));
  if (src_slot) {
    const int st = dtype == MOE_BF16 ? zero_pads<uint16_t>(src_slot, n_rows, d, x_perm, stream)
                                     : zero_pads<float>(src_slot, n_rows, d, x_perm, stream);
    if (st) return st;
  }
  if (T == 0) return MOE_OK;
  if (dtype == MOE_BF16)
    permute_kernel<uint16_t><<<row_grid(T), kRowThreads, 0, stream>>>(
        static_cast<const uint16_t*>(x), T, d, k, row_of, n_rows, static_cast<uint16_t*>(x_perm));
  else
    permute_kernel<float><<<row_grid(T), kRowThreads, 0, stream>>>(
        static_cast<const float*>(x), T, d, k, row_of, n_rows, static_cast<float*>(x_perm));
  return launch_status();
}

extern "C" int moe_unpermute_combine(int dtype, const void* y_perm, const int32_t* row_of,
                                     const float* topk_w, int T, int k, int d, int n_rows,
                                     const void* y_add, void* y, hipStream_t stream) {
  if (int st = check_rows(dtype, T, d, k, n_rows)) return st;
  if (T == 0) return MOE_OK;
  MOE_CHECK_ARG(row_of && topk_w && y && aligned16(y) && (n_rows == 0 || (y_perm && aligned16(y_perm))));
  MOE_CHECK_ARG(!y_add || aligned16(y_add));
  if (dtype == MOE_BF16)
    combine_kernel<uint16_t><<<row_grid(T), kRowThreads, 0, stream>>>(
        static_cast<const uint16_t*>(y_perm), row_of, topk_w, T, k, d, n_rows,
        static_cast<const uint16_t*>(y_add), static_cast<uint16_t*>(y));
  else
    combine_kernel<float><<<row_grid(T), kRowThreads, 0, stream>>>(
        static_cast<const float*>(y_perm), row_of, topk_w, T, k, d, n_rows,
        static_cast<const float*>(y_add), static_cast<float*>(y));
  return launch_status();
}

extern "C" int moe_unpermute_combine_bwd(int dtype, const void* dy, const void* y_perm,
                                         const float* topk_w, const int32_t* row_of,
                                         const int32_t* src_slot, int T, int k, int d, int n_rows,
                                         void* dy_perm, float* dtopk_w, hipStream_t stream) {
  if (int st = check_rows(dtype, T, d, k, n_rows)) return st;
  MOE_CHECK_ARG(src_slot || (long)n_rows == (long)T * k);
  MOE_CHECK_ARG(T == 0 || (dy && aligned16(dy) && topk_w && row_of && dtopk_w));
  MOE_CHECK_ARG(n_rows == 0 || (y_perm && dy_perm && aligned16(y_perm) && aligned16(dy_perm)));
  if (src_slot) {
    // row order: one wave per routed row, then one thread per slot
    const long row_blocks = ((long)n_rows * 64 + kRowThreads - 1) / kRowThreads;
    const long grid = row_blocks + ((long)T * k + kRowThreads - 1) / kRowThreads;
    if (grid == 0) return MOE_OK;
    MOE_CHECK_SUPPORTED(grid < (1L << 31));
    if (dtype == MOE_BF16)
      combine_bwd_rows_kernel<uint16_t><<<(int)grid, kRowThreads, 0, stream>>>(
          static_cast<const uint16_t*>(dy), static_cast<const uint16_t*>(y_perm), topk_w, row_of, src_slot, T,
          k, d, n_rows, (int)row_blocks, static_cast<uint16_t*>(dy_perm), dtopk_w);
    else
      combine_bwd_rows_kernel<float><<<(int)grid, kRowThreads, 0, stream>>>(
          static_cast<const float*>(dy), static_cast<const float*>(y_perm), topk_w, row_of, src_slot, T, k,
          d, n_rows, (int)row_blocks, static_cast<float*>(dy_perm), dtopk_w);
    return launch_status();
  }
  if (T == 0) return MOE_OK;
  if (dtype == MOE_BF16)
    combine_bwd_kernel<uint16_t><<<row_grid(T), kRowThreads, 0, stream>>>(
        static_cast<const uint16_t*>(dy), static_cast<const uint16_t*>(y_perm), topk_w, row_of, T,
        k, d, n_rows, static_cast<uint16_t*>(dy_perm), dtopk_w);
  else
    combine_bwd_kernel<float><<<row_grid(T), kRowThreads, 0, stream>>>(
        static_cast<const float*>(dy), static_cast<const float*>(y_perm), topk_w, row_of, T, k, d,
        n_rows, static_cast<float*>(dy_perm), dtopk_w);
  return launch_status();
}

extern "C" int moe_permute_bwd(int dtype, const void* dx_perm, const int32_t* row_of, int T, int k,
                               int d, int n_rows, const float* dlogits, const void* w_r, int E,
                               const void* dx_add, void* dx, hipStream_t stream) {
  if (int st = check_rows(dtype, T, d, k, n_rows)) return st;
  MOE_CHECK_ARG((dlogits == nullptr) == (w_r == nullptr));
  MOE_CHECK_ARG(!dlogits || (E > 0 && E <= MOE_MAX_EXPERTS && aligned16(w_r)));
  if (T == 0) return MOE_OK;
  MOE_CHECK_ARG(row_of && dx && aligned16(dx) && (n_rows == 0 || (dx_perm && aligned16(dx_perm))));
  MOE_CHECK_ARG(!dx_add || aligned16(dx_add));
  if (dtype == MOE_BF16)
    permute_bwd_kernel<uint16_t><<<row_grid(T), kRowThreads, 0, stream>>>(
        static_cast<const uint16_t*>(dx_perm), row_of, T, k, d, n_rows, dlogits,
        static_cast<const uint16_t*>(w_r), E, static_cast<const uint16_t*>(dx_add), static_cast<uint16_t*>(dx));
  else
    permute_bwd_kernel<float><<<row_grid(T), kRowThreads, 0, stream>>>(
        static_cast<const float*>(dx_perm), row_of, T, k, d, n_rows, dlogits,
        static_cast<const float*>(w_r), E, static_cast<const float*>(dx_add), static_cast<float*>(dx));
  return launch_status();
}
