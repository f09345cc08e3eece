// Grouped expert GEMMs (gfx950): the six GEMMs of a SwiGLU expert layer's
// forward and backward over uneven per-expert row blocks whose sizes live on
// the device only ("device-scheduled grouped GEMM", deniz.in, "Yeni stack
// nasıl çalışıyor").
//
// gg_mfma_kernel: bf16 operands, binary32 accumulation on the matrix cores
// (v_mfma_f32_32x32x16_bf16). A 128 x 256 output tile per workgroup of four
// waves (2 x 2, each wave 64 x 128), K staged through LDS in steps of 64 with
// double buffering. Both operands reach the matrix cores K-contiguous:
// operands that are contiguous along M or N in memory (weights in the
// forward pass, every operand of the weight gradients) are transposed in
// registers, four K-rows at a time, on their way into LDS. LDS rows are 128 B
// with the 16-byte chunk index XOR-swizzled by the row so that both the
// transposed writes and the fragment reads avoid bank conflicts.
//
// gg_simple_kernel: any dtype and shape, binary32 FMA on 64 x 64 tiles; it
// serves binary32 layers and shapes outside the MFMA kernel's limits.
#include "gemm_common.h"

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
      Elem<T>::store((T*)a.g, i, g);
      Elem<T>::store((T*)a.u, i, u);
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

// ======================================================================== MFMA kernel
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

constexpr int kBM = 128;    // output rows per tile
constexpr int kBN = 256;    // LDS n-rows per tile (128 + 128 for the dual ops)
constexpr int kBK = 64;     // K step
constexpr int kNT = 256;    // threads

// 16-byte chunk swizzle of LDS row r (rows are kBK = 64 bf16 = 8 chunks).
MOE_DEV int swz(int r) { return (r ^ (r >> 3)) & 7; }
MOE_DEV int lds_off(int row, int chunk) { return row * kBK + ((chunk ^ swz(row)) << 3); }

MOE_DEV V16 zero16() {
  V16 z;
#pragma unroll
  for (int i = 0; i < 4; ++i) z.w[i] = 0u;
  return z;
}

// Store 4 K-rows x 8 MN-columns (one V16 per K-row) as 8 LDS rows (one per
// MN column) of 4 K-values, at K-quad kq of the 64-wide row.
MOE_DEV void store_transposed(uint16_t* s, int row0, int kq, const V16 (&r)[4]) {
#pragma unroll
  for (int mm = 0; mm < 8; ++mm) {
    const int w = mm >> 1;
    const bool hi = mm & 1;
    auto pick = [&](const V16& v) -> uint32_t { return hi ? (v.w[w] >> 16) : (v.w[w] & 0xffffu); };
    uint2 o;
    o.x = pick(r[0]) | (pick(r[1]) << 16);
    o.y = pick(r[2]) | (pick(r[3]) << 16);
    const int row = row0 + mm;
    *reinterpret_cast<uint2*>(s + row * kBK + ((((kq >> 1) ^ swz(row)) << 3) + (kq & 1) * 4)) = o;
  }
}

template <int OP>
__global__ void __launch_bounds__(kNT, 1) gg_mfma_kernel(GGArgs a) {
  using I = OpInfo<OP>;
  constexpr bool DUAL = I::kDual, KVAR = I::kKVar, AK = I::kAKContig, BKC = I::kBKContig;
  constexpr int BNO = DUAL ? kBN / 2 : kBN;   // output columns per matrix per tile
  __shared__ int tile_start[MOE_MAX_EXPERTS + 1];
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][kBM * kBK];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][kBN * kBK];

  const int d = a.d, F = a.F;
  const int N = op_n(OP, d, F);
  const int tilesN = N / BNO;
  const int b = xcd_remap(blockIdx.x, gridDim.x);
  int e, row0, mv, K, m0 = 0, tn;
  if (!KVAR) {
    tn = b % tilesN;
    if (!find_m_tile<kBM, kNT>(a, b / tilesN, tile_start, e, row0, mv)) return;
    K = op_k(OP, d, F);
  } else {
    const int M = op_wgrad_m(OP, d, F);
    const int per = (M / kBM) * tilesN;
    e = b / per;
    m0 = ((b % per) / tilesN) * kBM;
    tn = b % tilesN;
    group_rows(a, e, row0, K);
    mv = kBM;
  }
  const int n0 = tn * BNO;
  const size_t dF = (size_t)d * F;
  const uint16_t* Ab = nullptr;        // A base at (row 0 or m0, k 0)
  const uint16_t* Bb[2] = {nullptr, nullptr};
  int lda = 0, ldb = 0;
  switch (OP) {
    case MOE_GG_FWD_GATE_UP:
      Ab = (const uint16_t*)a.x_perm + (size_t)row0 * d; lda = d;
      Bb[0] = (const uint16_t*)a.w_gate + e * dF + n0;
      Bb[1] = (const uint16_t*)a.w_up + e * dF + n0; ldb = F;
      break;
    case MOE_GG_FWD_DOWN:
      Ab = (const uint16_t*)a.h + (size_t)row0 * F; lda = F;
      Bb[0] = (const uint16_t*)a.w_down + e * dF + n0; ldb = d;
      break;
    case MOE_GG_DGRAD_DOWN:
      Ab = (const uint16_t*)a.dy_perm + (size_t)row0 * d; lda = d;
      Bb[0] = (const uint16_t*)a.w_down + e * dF + (size_t)n0 * d; ldb = d;
      break;
    case MOE_GG_DGRAD_GATE_UP:
      Ab = (const uint16_t*)a.dg + (size_t)row0 * F; lda = F;
      Bb[0] = (const uint16_t*)a.w_gate + e * dF + (size_t)n0 * F;
      Bb[1] = (const uint16_t*)a.w_up + e * dF + (size_t)n0 * F; ldb = F;
      break;
    case MOE_GG_WGRAD_DOWN:
      Ab = (const uint16_t*)a.h + (size_t)row0 * F + m0; lda = F;
      Bb[0] = (const uint16_t*)a.dy_perm + (size_t)row0 * d + n0; ldb = d;
      break;
    default:   // WGRAD_GATE_UP
      Ab = (const uint16_t*)a.x_perm + (size_t)row0 * d + m0; lda = d;
      Bb[0] = (const uint16_t*)a.dg + (size_t)row0 * F + n0;
      Bb[1] = (const uint16_t*)a.du + (size_t)row0 * F + n0; ldb = F;
  }
  const uint16_t* Ab2 = OP == MOE_GG_DGRAD_GATE_UP ? (const uint16_t*)a.du + (size_t)row0 * F : nullptr;

  const int tid = threadIdx.x;
  V16 ra[4], rb[8];

  // ---- global -> registers
  auto load = [&](int k0) {
    if (AK) {
      const uint16_t* A = Ab;
      int kc0 = k0;
      if (OP == MOE_GG_DGRAD_GATE_UP && k0 >= F) { A = Ab2; kc0 = k0 - F; }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int q = i * kNT + tid, m = q >> 3, kc = q & 7;
        ra[i] = m < mv ? *reinterpret_cast<const V16*>(A + (size_t)m * lda + kc0 + kc * 8) : zero16();
      }
    } else {
      const int o = tid & 15, kq = tid >> 4;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int kk = k0 + 4 * kq + ii;
        ra[ii] = kk < K ? *reinterpret_cast<const V16*>(Ab + (size_t)kk * lda + 8 * o) : zero16();
      }
    }
    if (BKC) {
      const uint16_t* B = Bb[0];
      int kc0 = k0;
      if (OP == MOE_GG_DGRAD_GATE_UP && k0 >= F) { B = Bb[1]; kc0 = k0 - F; }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int q = i * kNT + tid, n = q >> 3, kc = q & 7;
        rb[i] = *reinterpret_cast<const V16*>(B + (size_t)n * ldb + kc0 + kc * 8);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int u = i * kNT + tid, o = u & 31, kq = u >> 5;
        const int r = 8 * o;
        int col = r, mat = 0;
        if (DUAL) { mat = (r & 127) >> 6; col = (r >> 7) * 64 + (r & 63); }
        const uint16_t* B = Bb[mat];
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int kk = k0 + 4 * kq + ii;
          const bool ok = !KVAR || kk < K;
          rb[i * 4 + ii] = ok ? *reinterpret_cast<const V16*>(B + (size_t)kk * ldb + col) : zero16();
        }
      }
    }
  };
  // ---- registers -> LDS
  auto store = [&](int buf) {
    uint16_t* A = sA[buf];
    uint16_t* B = sB[buf];
    if (AK) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int q = i * kNT + tid, m = q >> 3, kc = q & 7;
        *reinterpret_cast<V16*>(A + lds_off(m, kc)) = ra[i];
      }
    } else {
      const int o = tid & 15, kq = tid >> 4;
      store_transposed(A, 8 * o, kq, ra);
    }
    if (BKC) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int q = i * kNT + tid, n = q >> 3, kc = q & 7;
        *reinterpret_cast<V16*>(B + lds_off(n, kc)) = rb[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int u = i * kNT + tid, o = u & 31, kq = u >> 5;
        const V16 r4[4] = {rb[i * 4], rb[i * 4 + 1], rb[i * 4 + 2], rb[i * 4 + 3]};
        store_transposed(B, 8 * o, kq, r4);
      }
    }
  };

  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, lk = lane >> 5;
  f32x16_t acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = (K + kBK - 1) / kBK;
  if (nk > 0) {
    load(0);
    store(0);
  }
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load((kt + 1) * kBK);
    const uint16_t* A = sA[cur];
    const uint16_t* B = sB[cur];
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      bf16x8_t af[2], bfr[4];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        const int row = wm * 64 + mi * 32 + lr;
        af[mi] = *reinterpret_cast<const bf16x8_t*>(A + lds_off(row, 2 * kk + lk));
      }
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        const int row = wn * 128 + ni * 32 + lr;
        bfr[ni] = *reinterpret_cast<const bf16x8_t*>(B + lds_off(row, 2 * kk + lk));
      }
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[ni], af[mi], acc[mi][ni], 0, 0, 0);
    }
    if (kt + 1 < nk) store(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds row m = lr of each 32-row block and, per group g
  // of 4 accumulators, 4 consecutive output columns 8g + 4lk .. +3.
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
    const int ml = wm * 64 + mi * 32 + lr;
    if (ml >= mv) continue;
    const size_t row = KVAR ? (size_t)(m0 + ml) : (size_t)(row0 + ml);
#pragma unroll
    for (int ni = 0; ni < (DUAL ? 2 : 4); ++ni) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int cl = ni * 32 + 8 * g + 4 * lk;
        float v0[4], v1[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          v0[r] = acc[mi][ni][4 * g + r];
          v1[r] = DUAL ? acc[mi][ni + 2][4 * g + r] : 0.f;
        }
        if (OP == MOE_GG_FWD_GATE_UP) {
          const size_t i = row * F + n0 + wn * 64 + cl;
          float gg[4], uu[4], hh[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) swiglu_fwd<uint16_t>(v0[r], v1[r], gg[r], uu[r], hh[r]);
          *reinterpret_cast<uint2*>((uint16_t*)a.g + i) = make_uint2(pack_bf16x2(gg[0], gg[1]), pack_bf16x2(gg[2], gg[3]));
          *reinterpret_cast<uint2*>((uint16_t*)a.u + i) = make_uint2(pack_bf16x2(uu[0], uu[1]), pack_bf16x2(uu[2], uu[3]));
          *reinterpret_cast<uint2*>((uint16_t*)a.h + i) = make_uint2(pack_bf16x2(hh[0], hh[1]), pack_bf16x2(hh[2], hh[3]));
        } else if (OP == MOE_GG_WGRAD_GATE_UP) {
          const size_t i = e * dF + row * F + n0 + wn * 64 + cl;
          *reinterpret_cast<uint2*>((uint16_t*)a.dw_gate + i) = make_uint2(pack_bf16x2(v0[0], v0[1]), pack_bf16x2(v0[2], v0[3]));
          *reinterpret_cast<uint2*>((uint16_t*)a.dw_up + i) = make_uint2(pack_bf16x2(v1[0], v1[1]), pack_bf16x2(v1[2], v1[3]));
        } else if (OP == MOE_GG_DGRAD_DOWN) {
          const size_t i = row * F + n0 + wn * 128 + cl;
          const uint2 gv = *reinterpret_cast<const uint2*>((const uint16_t*)a.g + i);
          const uint2 uv = *reinterpret_cast<const uint2*>((const uint16_t*)a.u + i);
          const float gf[4] = {__uint_as_float(gv.x << 16), __uint_as_float(gv.x & 0xffff0000u),
                               __uint_as_float(gv.y << 16), __uint_as_float(gv.y & 0xffff0000u)};
          const float uf[4] = {__uint_as_float(uv.x << 16), __uint_as_float(uv.x & 0xffff0000u),
                               __uint_as_float(uv.y << 16), __uint_as_float(uv.y & 0xffff0000u)};
          float dg[4], du[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) swiglu_bwd(v0[r], gf[r], uf[r], dg[r], du[r]);
          *reinterpret_cast<uint2*>((uint16_t*)a.dg + i) = make_uint2(pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3]));
          *reinterpret_cast<uint2*>((uint16_t*)a.du + i) = make_uint2(pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3]));
        } else {
          uint16_t* out;
          size_t i;
          if (OP == MOE_GG_FWD_DOWN) { out = (uint16_t*)a.y_perm; i = row * d; }
          else if (OP == MOE_GG_DGRAD_GATE_UP) { out = (uint16_t*)a.dx_perm; i = row * d; }
          else { out = (uint16_t*)a.dw_down; i = e * dF + row * d; }
          i += n0 + wn * 128 + cl;
          *reinterpret_cast<uint2*>(out + i) = make_uint2(pack_bf16x2(v0[0], v0[1]), pack_bf16x2(v0[2], v0[3]));
        }
      }
    }
  }
}

}  // namespace moe

// ======================================================================== C ABI
using namespace moe;

namespace {

bool mfma_ok(const moe_gg_desc* g) {
  return g->dtype == MOE_BF16 && g->d % kBN == 0 && g->F % kBN == 0;
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

template <int OP> struct LaunchMfma {
  static void go(const GGArgs& a, int grid, hipStream_t s) {
    gg_mfma_kernel<OP><<<grid, kNT, 0, s>>>(a);
  }
};
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

extern "C" size_t moe_grouped_gemm_workspace_bytes(const moe_gg_desc* desc) {
  (void)desc;
  return 0;
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
  auto need = [](const void* p) { return p != nullptr && aligned16(p); };
  switch (g->op) {
    case MOE_GG_FWD_GATE_UP:
      MOE_CHECK_ARG(need(g->x_perm) && need(g->w_gate) && need(g->w_up) && need(g->g) && need(g->u) && need(g->h));
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
      MOE_CHECK_ARG(need(g->h) && need(g->dy_perm) && need(g->dw_down));
      break;
    default:
      MOE_CHECK_ARG(need(g->x_perm) && need(g->dg) && need(g->du) && need(g->dw_gate) && need(g->dw_up));
  }
  GGArgs a{g->op, g->E, g->d, g->F, g->n_rows, g->capacity, g->group_offsets,
           g->x_perm, g->g, g->u, g->h, g->y_perm, g->dy_perm, g->dg, g->du, g->dx_perm,
           g->w_gate, g->w_up, g->w_down, g->dw_gate, g->dw_up, g->dw_down};
  const bool kvar = g->op == MOE_GG_WGRAD_DOWN || g->op == MOE_GG_WGRAD_GATE_UP;
  const bool dual = g->op == MOE_GG_FWD_GATE_UP || g->op == MOE_GG_WGRAD_GATE_UP;
  const int N = op_n(g->op, g->d, g->F);
  if (mfma_ok(g)) {
    const int bno = dual ? kBN / 2 : kBN;
    long grid;
    if (kvar) grid = (long)g->E * (op_wgrad_m(g->op, g->d, g->F) / kBM) * (N / bno);
    else grid = (cdiv(g->n_rows, kBM) + g->E) * (N / bno);
    if (grid == 0) return MOE_OK;
    MOE_CHECK_SUPPORTED(grid < (1L << 31));
    return dispatch_op<LaunchMfma>(g->op, a, static_cast<int>(grid), stream);
  }
  long grid;
  if (kvar) grid = (long)g->E * cdiv(op_wgrad_m(g->op, g->d, g->F), kSBM) * cdiv(N, kSBN);
  else grid = (cdiv(g->n_rows, kSBM) + g->E) * cdiv(N, kSBN);
  if (grid == 0) return MOE_OK;
  MOE_CHECK_SUPPORTED(grid < (1L << 31));
  if (g->dtype == MOE_BF16) return dispatch_op<LaunchSimpleBf16>(g->op, a, static_cast<int>(grid), stream);
  return dispatch_op<LaunchSimpleF32>(g->op, a, static_cast<int>(grid), stream);
}
