// Grouped expert GEMMs (gfx950): the six GEMMs of a SwiGLU expert layer's
// forward and backward over uneven per-expert row blocks whose sizes live on
// the device only ("device-scheduled grouped GEMM", deniz.in, "Yeni stack
// nasıl çalışıyor").
//
// gg_dma_kernel (gemm_dma.h): bf16 operands, binary32 accumulation on the
// matrix cores, tiles loaded straight from memory into LDS, an on-device
// group-tile scheduler.
//
// gg_simple_kernel: any dtype and shape, binary32 FMA on 64 x 64 tiles; it
// serves binary32 layers and shapes outside the MFMA kernel's limits.
#include "gemm_dma.h"

namespace moe {

// ======================================================================== shared semantics
template <typename T> MOE_DEV float rnd(float v);
template <> MOE_DEV float rnd<float>(float v) { return v; }
template <> MOE_DEV float rnd<uint16_t>(float v) { return bf16_to_f32(f32_to_bf16(v)); }

// SwiGLU forward from the stored (rounded) g and u.
template <typename T> MOE_DEV void swiglu_fwd(float acc_g, float acc_u, float& g, float& u, float& h) {
  g = rnd<T>(acc_g);
  u = rnd<T>(acc_u);
  h = g * u / (1.0f + expf(-g));
}
// SwiGLU backward: dg = dh*u*s*(1+g*(1-s)), du = dh*g*s with s = sigmoid(g).
MOE_DEV void swiglu_bwd(float dh, float g, float u, float& dg, float& du) {
  const float s = 1.0f / (1.0f + expf(-g));
  dg = dh * u * s * (1.0f + g * (1.0f - s));
  du = dh * g * s;
}

// ======================================================================== plain FMA kernel
constexpr int kSBM = 64, kSBN = 64, kSBK = 16;

template <typename T, int OP>
MOE_DEV float simple_a(const GGArgs& a, int e, int row0, int m0, int m, int k) {
  const int d = a.d, F = a.F;
  switch (OP) {
    case MOE_GG_FWD_GATE_UP: return Elem<T>::load((const T*)a.x_perm, (size_t)(row0 + m) * d + k);
    case MOE_GG_FWD_DOWN: return Elem<T>::load((const T*)a.h, (size_t)(row0 + m) * F + k);
    case MOE_GG_DGRAD_DOWN: return Elem<T>::load((const T*)a.dy_perm, (size_t)(row0 + m) * d + k);
    case MOE_GG_DGRAD_GATE_UP:
      return k < F ? Elem<T>::load((const T*)a.dg, (size_t)(row0 + m) * F + k)
                   : Elem<T>::load((const T*)a.du, (size_t)(row0 + m) * F + (k - F));
    case MOE_GG_WGRAD_DOWN: return Elem<T>::load((const T*)a.h, (size_t)(row0 + k) * F + m0 + m);
    default: return Elem<T>::load((const T*)a.x_perm, (size_t)(row0 + k) * d + m0 + m);
  }
}

template <typename T, int OP>
MOE_DEV float simple_b(const GGArgs& a, int e, int row0, int k, int n, int which) {
  const size_t d = a.d, F = a.F;
  switch (OP) {
    case MOE_GG_FWD_GATE_UP:
      return Elem<T>::load((const T*)(which ? a.w_up : a.w_gate), e * d * F + k * F + n);
    case MOE_GG_FWD_DOWN: return Elem<T>::load((const T*)a.w_down, e * F * d + k * d + n);
    case MOE_GG_DGRAD_DOWN: return Elem<T>::load((const T*)a.w_down, e * F * d + n * d + k);
    case MOE_GG_DGRAD_GATE_UP:
      return (size_t)k < F ? Elem<T>::load((const T*)a.w_gate, e * d * F + n * F + k)
                           : Elem<T>::load((const T*)a.w_up, e * d * F + n * F + (k - F));
    case MOE_GG_WGRAD_DOWN: return Elem<T>::load((const T*)a.dy_perm, (size_t)(row0 + k) * d + n);
    default:
      return Elem<T>::load((const T*)(which ? a.du : a.dg), (size_t)(row0 + k) * F + n);
  }
}

// Epilogue of one output element; row is the permuted row (row-varying ops)
// or the weight row (weight gradients).
template <typename T, int OP>
MOE_DEV void simple_store(const GGArgs& a, int e, int row, int n, float c0, float c1) {
  const size_t d = a.d, F = a.F;
  switch (OP) {
    case MOE_GG_FWD_GATE_UP: {
      float g, u, h;
      swiglu_fwd<T>(c0, c1, g, u, h);
      const size_t i = (size_t)row * F + n;
      if (a.g != nullptr) {   // null g and u: only h is written (recompute)
        Elem<T>::store((T*)a.g, i, g);
        Elem<T>::store((T*)a.u, i, u);
      }
      Elem<T>::store((T*)a.h, i, h);
      break;
    }
    case MOE_GG_FWD_DOWN: Elem<T>::store((T*)a.y_perm, (size_t)row * d + n, c0); break;
    case MOE_GG_DGRAD_DOWN: {
      const size_t i = (size_t)row * F + n;
      float dg, du;
      swiglu_bwd(c0, Elem<T>::load((const T*)a.g, i), Elem<T>::load((const T*)a.u, i), dg, du);
      Elem<T>::store((T*)a.dg, i, dg);
      Elem<T>::store((T*)a.du, i, du);
      break;
    }
    case MOE_GG_DGRAD_GATE_UP: Elem<T>::store((T*)a.dx_perm, (size_t)row * d + n, c0); break;
    case MOE_GG_WGRAD_DOWN: Elem<T>::store((T*)a.dw_down, e * F * d + (size_t)row * d + n, c0); break;
    default:
      Elem<T>::store((T*)a.dw_gate, e * d * F + (size_t)row * F + n, c0);
      Elem<T>::store((T*)a.dw_up, e * d * F + (size_t)row * F + n, c1);
  }
}

template <typename T, int OP>
__global__ void __launch_bounds__(256) gg_simple_kernel(GGArgs a) {
  using I = OpInfo<OP>;
  __shared__ int tile_start[MOE_MAX_EXPERTS + 1];
  __shared__ float As[kSBK][kSBM + 1];
  __shared__ float Bs[2][kSBK][kSBN + 1];
  const int N = op_n(OP, a.d, a.F);
  const int tilesN = (N + kSBN - 1) / kSBN;
  int e, row0, mv, K, m0 = 0, tn;
  if (!I::kKVar) {
    const int tm = blockIdx.x / tilesN;
    tn = blockIdx.x % tilesN;
    if (!find_m_tile<kSBM, 256>(a, tm, tile_start, e, row0, mv)) return;
    K = op_k(OP, a.d, a.F);
  } else {
    const int M = op_wgrad_m(OP, a.d, a.F);
    const int tilesM = (M + kSBM - 1) / kSBM;
    e = blockIdx.x / (tilesM * tilesN);
    const int rem = blockIdx.x % (tilesM * tilesN);
    m0 = (rem / tilesN) * kSBM;
    tn = rem % tilesN;
    group_rows(a, e, row0, K);
    mv = min(kSBM, M - m0);
  }
  const int n0 = tn * kSBN;
  const int nv = min(kSBN, N - n0);
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  float c[2][4][4] = {};
  for (int k0 = 0; k0 < K; k0 += kSBK) {
    for (int i = threadIdx.x; i < kSBK * kSBM; i += 256) {
      const int kk = i / kSBM, m = i % kSBM;
      As[kk][m] = (m < mv && k0 + kk < K) ? simple_a<T, OP>(a, e, row0, m0, m, k0 + kk) : 0.f;
    }
    for (int i = threadIdx.x; i < kSBK * kSBN; i += 256) {
      const int kk = i / kSBN, n = i % kSBN;
      const bool ok = n < nv && k0 + kk < K;
      Bs[0][kk][n] = ok ? simple_b<T, OP>(a, e, row0, k0 + kk, n0 + n, 0) : 0.f;
      if (I::kDual) Bs[1][kk][n] = ok ? simple_b<T, OP>(a, e, row0, k0 + kk, n0 + n, 1) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kSBK; ++kk) {
      float av[4], bv[2][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[kk][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bv[0][j] = Bs[0][kk][tx + 16 * j];
        bv[1][j] = I::kDual ? Bs[1][kk][tx + 16 * j] : 0.f;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          c[0][i][j] = fmaf(av[i], bv[0][j], c[0][i][j]);
          if (I::kDual) c[1][i][j] = fmaf(av[i], bv[1][j], c[1][i][j]);
        }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = ty + 16 * i, n = tx + 16 * j;
      if (m < mv && n < nv)
        simple_store<T, OP>(a, e, I::kKVar ? m0 + m : row0 + m, n0 + n, c[0][i][j], c[1][i][j]);
    }
}

}  // namespace moe

// ======================================================================== C ABI
using namespace moe;

namespace {

// The direct-load kernel on 128 x 256 tiles, eight waves of 64 x 64 and two
// workgroups per CU (16 waves per CU hide the per-stage load issue, fragment
// reads and barriers of each other).
using CfgDma = DmaCfg<128, 256, 2, 4, 32, 3, 2>;

bool mfma_ok(const moe_gg_desc* g) {
  return g->dtype == MOE_BF16 && g->d % 256 == 0 && g->F % 256 == 0;
}

template <template <int> class Launch>
int dispatch_op(int op, const GGArgs& a, int grid, hipStream_t s) {
  switch (op) {
    case MOE_GG_FWD_GATE_UP: Launch<MOE_GG_FWD_GATE_UP>::go(a, grid, s); break;
    case MOE_GG_FWD_DOWN: Launch<MOE_GG_FWD_DOWN>::go(a, grid, s); break;
    case MOE_GG_DGRAD_DOWN: Launch<MOE_GG_DGRAD_DOWN>::go(a, grid, s); break;
    case MOE_GG_DGRAD_GATE_UP: Launch<MOE_GG_DGRAD_GATE_UP>::go(a, grid, s); break;
    case MOE_GG_WGRAD_DOWN: Launch<MOE_GG_WGRAD_DOWN>::go(a, grid, s); break;
    default: Launch<MOE_GG_WGRAD_GATE_UP>::go(a, grid, s); break;
  }
  return launch_status();
}

template <class C> struct Dma {
  template <int OP> struct Launch {
    static void go(const GGArgs& a, int grid, hipStream_t s) {
      gg_dma_kernel<OP, C><<<grid, C::NT, 0, s>>>(a);
    }
  };
};

template <int OP> struct SplitReduce {
  static void go(const GGArgs& a, int grid, hipStream_t s) {
    if constexpr (OpInfo<OP>::kKVar) gg_splitk_reduce_kernel<OP><<<grid, 256, 0, s>>>(a);
  }
};

template <class C> struct DmaSplit {
  template <int OP> struct Launch {
    static void go(const GGArgs& a, int grid, hipStream_t s) {
      if constexpr (OpInfo<OP>::kKVar)
        gg_wgrad_split_kernel<OP, C><<<1, 256, 0, s>>>(a, grid, const_cast<int*>(a.split));
    }
  };
};

template <class C>
int launch_dma(const moe_gg_desc* g, const GGArgs& a, bool kvar, bool dual, int N, hipStream_t stream) {
  const int bno = dual ? C::BN / 2 : C::BN;
  long grid;
  if (kvar) grid = (long)g->E * (op_wgrad_m(g->op, g->d, g->F) / C::BM) * (N / bno);
  else grid = ((g->n_rows + C::BM - 1) / C::BM + g->E) * (long)(N / bno);
  if (grid == 0) return MOE_OK;
  MOE_CHECK_SUPPORTED(grid * (a.ksplit > 1 ? a.ksplit : 1) < (1L << 31));
  if (a.ksplit > 1) {   // K split into chunks, then the ordered reduction of their partial sums
    const long nout = (long)g->E * op_wgrad_m(g->op, g->d, g->F) * N * (dual ? 2 : 1);
    if (int st = dispatch_op<Dma<C>::template Launch>(g->op, a, static_cast<int>(grid * a.ksplit), stream)) return st;
    return dispatch_op<SplitReduce>(g->op, a, static_cast<int>((nout / 8 + 255) / 256), stream);
  }
  if (kvar && a.split) {   // the launch's tile split, from the device-resident group sizes
    if (int st = dispatch_op<DmaSplit<C>::template Launch>(g->op, a, static_cast<int>(grid), stream)) return st;
  }
  return dispatch_op<Dma<C>::template Launch>(g->op, a, static_cast<int>(grid), stream);
}

template <int OP> struct LaunchSimpleBf16 {
  static void go(const GGArgs& a, int grid, hipStream_t s) {
    gg_simple_kernel<uint16_t, OP><<<grid, 256, 0, s>>>(a);
  }
};
template <int OP> struct LaunchSimpleF32 {
  static void go(const GGArgs& a, int grid, hipStream_t s) {
    gg_simple_kernel<float, OP><<<grid, 256, 0, s>>>(a);
  }
};

long cdiv(long a, long b) { return (a + b - 1) / b; }

}  // namespace

// Weight gradients over device-resident groups keep their launch's tile
// split (kSplitInts ints) in the workspace.
constexpr size_t kSplitBytes = 64;
static_assert(kSplitInts * sizeof(int) <= kSplitBytes, "split fits the workspace");

// A weight-gradient launch of fewer tiles than this leaves CUs idle (two
// workgroups fit on each of the 256 CUs): its K (the expert's rows) is split
// into up to kMaxKSplit chunks whose binary32 partial sums start at byte
// kPartialOffset of the workspace.
constexpr long kSplitKTiles = 512;
constexpr int kMaxKSplit = 8;
constexpr size_t kPartialOffset = 256;

namespace {
bool is_kvar(int op) { return op == MOE_GG_WGRAD_DOWN || op == MOE_GG_WGRAD_GATE_UP; }

// K chunks of a weight-gradient launch (1: not split).
int wgrad_ksplit(const moe_gg_desc* g) {
  if (!is_kvar(g->op) || g->capacity != 0 || !mfma_ok(g)) return 1;
  const int bno = g->op == MOE_GG_WGRAD_GATE_UP ? CfgDma::BN / 2 : CfgDma::BN;
  const long tiles = (long)g->E * (op_wgrad_m(g->op, g->d, g->F) / CfgDma::BM) * (op_n(g->op, g->d, g->F) / bno);
  if (tiles >= kSplitKTiles) return 1;
  const long ks = (kSplitKTiles + tiles - 1) / tiles;
  return ks > kMaxKSplit ? kMaxKSplit : static_cast<int>(ks);
}

size_t splitk_bytes(const moe_gg_desc* g, int ks) {
  const size_t np = (size_t)op_n(g->op, g->d, g->F) * (g->op == MOE_GG_WGRAD_GATE_UP ? 2 : 1);
  return (size_t)ks * g->E * op_wgrad_m(g->op, g->d, g->F) * np * sizeof(float);
}
}  // namespace

extern "C" size_t moe_grouped_gemm_workspace_bytes(const moe_gg_desc* desc) {
  if (desc == nullptr || !is_kvar(desc->op) || desc->capacity != 0) return 0;
  if (desc->E < 1 || desc->d <= 0 || desc->F <= 0) return kSplitBytes;
  const int ks = wgrad_ksplit(desc);
  return ks > 1 ? kPartialOffset + splitk_bytes(desc, ks) : kSplitBytes;
}

extern "C" int moe_grouped_gemm(const moe_gg_desc* g, hipStream_t stream) {
  MOE_CHECK_ARG(g != nullptr);
  MOE_CHECK_ARG(valid_dtype(g->dtype) && g->op >= MOE_GG_FWD_GATE_UP && g->op <= MOE_GG_WGRAD_GATE_UP);
  MOE_CHECK_ARG(g->E >= 1 && g->d > 0 && g->F > 0 && g->n_rows >= 0 && g->capacity >= 0);
  MOE_CHECK_ARG(g->d % 8 == 0 && g->F % 8 == 0);
  MOE_CHECK_SUPPORTED(g->E <= MOE_MAX_EXPERTS);
  MOE_CHECK_SUPPORTED((long)g->n_rows * (g->d > g->F ? g->d : g->F) < (1L << 40));
  MOE_CHECK_ARG(g->capacity > 0 || g->group_offsets != nullptr);
  MOE_CHECK_ARG(g->capacity == 0 || (long)g->E * g->capacity <= g->n_rows);
  const bool kvar = g->op == MOE_GG_WGRAD_DOWN || g->op == MOE_GG_WGRAD_GATE_UP;
  // with no rows a row-varying op has nothing to do, and a weight gradient
  // reads no activations (every expert's gradient is zero)
  if (g->n_rows == 0 && !kvar) return MOE_OK;
  const bool rows = g->n_rows > 0;
  auto need = [](const void* p) { return p != nullptr && aligned16(p); };
  auto act = [&](const void* p) { return !rows || (p != nullptr && aligned16(p)); };
  switch (g->op) {
    case MOE_GG_FWD_GATE_UP:
      MOE_CHECK_ARG(need(g->x_perm) && need(g->w_gate) && need(g->w_up) && need(g->h));
      // g and u both written, or both NULL (only h is wanted)
      MOE_CHECK_ARG((need(g->g) && need(g->u)) || (g->g == nullptr && g->u == nullptr));
      break;
    case MOE_GG_FWD_DOWN:
      MOE_CHECK_ARG(need(g->h) && need(g->w_down) && need(g->y_perm));
      break;
    case MOE_GG_DGRAD_DOWN:
      MOE_CHECK_ARG(need(g->dy_perm) && need(g->w_down) && need(g->g) && need(g->u) && need(g->dg) && need(g->du));
      break;
    case MOE_GG_DGRAD_GATE_UP:
      MOE_CHECK_ARG(need(g->dg) && need(g->du) && need(g->w_gate) && need(g->w_up) && need(g->dx_perm));
      break;
    case MOE_GG_WGRAD_DOWN:
      MOE_CHECK_ARG(act(g->h) && act(g->dy_perm) && need(g->dw_down));
      break;
    default:
      MOE_CHECK_ARG(act(g->x_perm) && act(g->dg) && act(g->du) && need(g->dw_gate) && need(g->dw_up));
  }
  // the tile split needs kSplitBytes; a launch that would split K does so only
  // when the workspace also holds the partial sums (16-byte aligned)
  const size_t ws_need = kvar && g->capacity == 0 ? kSplitBytes : 0;
  if (ws_need > 0 && (g->ws == nullptr || g->ws_bytes < ws_need || !aligned4(g->ws))) return MOE_ERR_WORKSPACE;
  int ksplit = wgrad_ksplit(g);
  if (ksplit > 1 && (g->ws_bytes < kPartialOffset + splitk_bytes(g, ksplit) || !aligned16(g->ws))) ksplit = 1;
  GGArgs a{g->op, g->E, g->d, g->F, g->n_rows, g->capacity, g->group_offsets,
           g->x_perm, g->g, g->u, g->h, g->y_perm, g->dy_perm, g->dg, g->du, g->dx_perm,
           g->w_gate, g->w_up, g->w_down, g->dw_gate, g->dw_up, g->dw_down,
           ws_need > 0 ? static_cast<const int*>(g->ws) : nullptr};
  if (ksplit > 1) {
    a.partial = reinterpret_cast<float*>(static_cast<char*>(g->ws) + kPartialOffset);
    a.ksplit = ksplit;
  }
  const bool dual = g->op == MOE_GG_FWD_GATE_UP || g->op == MOE_GG_WGRAD_GATE_UP;
  const int N = op_n(g->op, g->d, g->F);
  if (mfma_ok(g)) {
    // buffer-resource offsets are 32-bit: every expert's rows and weights
    // must span less than 2 GiB
    const long span = (long)g->n_rows * (g->d > g->F ? g->d : g->F) * 2;
    MOE_CHECK_SUPPORTED(span < (1L << 31) && (long)g->d * g->F * 2 < (1L << 31));
    return launch_dma<CfgDma>(g, a, kvar, dual, N, stream);
  }
  long grid;
  if (kvar) grid = (long)g->E * cdiv(op_wgrad_m(g->op, g->d, g->F), kSBM) * cdiv(N, kSBN);
  else grid = (cdiv(g->n_rows, kSBM) + g->E) * cdiv(N, kSBN);
  if (grid == 0) return MOE_OK;
  MOE_CHECK_SUPPORTED(grid < (1L << 31));
  if (g->dtype == MOE_BF16) return dispatch_op<LaunchSimpleBf16>(g->op, a, static_cast<int>(grid), stream);
  return dispatch_op<LaunchSimpleF32>(g->op, a, static_cast<int>(grid), stream);
}
