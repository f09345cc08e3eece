// bf16 grouped expert GEMM on the CDNA4 matrix cores (v_mfma_f32_32x32x16_bf16).
//
// One workgroup computes a BM x BN tile of one expert (BN counts LDS n-rows:
// for the dual ops half of them are gate columns and half are up columns).
// WM x WN wave64s each own a (BM/WM) x (BN/WN) sub-tile of 32 x 32 MFMA
// blocks. K advances 64 at a time through double-buffered LDS; the next step's
// global loads are in flight while the current step computes. Both operands
// reach the matrix cores K-contiguous: operands contiguous along M or N in
// memory are transposed in registers four K-rows at a time on their way into
// LDS. LDS rows are 128 B; the 16-byte chunk index is XOR-swizzled by
// (row ^ row >> 3) & 7 so that fragment reads (8 consecutive rows, same
// chunk) and transposed writes (rows 8 apart) both spread over the banks.
#pragma once

#include "gemm_common.h"

namespace moe {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

constexpr int kBK = 64;   // K step (elements)

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
MOE_DEV void store_transposed(uint16_t* s, int row0, int kq, const V16* r) {
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

MOE_DEV uint2 pack4(const float* v) { return make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])); }
MOE_DEV void unpack4(uint2 p, float* v) {
  v[0] = __uint_as_float(p.x << 16);
  v[1] = __uint_as_float(p.x & 0xffff0000u);
  v[2] = __uint_as_float(p.y << 16);
  v[3] = __uint_as_float(p.y & 0xffff0000u);
}

// Tile shape of the MFMA kernel.
template <int BM_, int BN_, int WM_, int WN_> struct MfmaCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int NT = WM * WN * 64;
  static constexpr int WMR = BM / WM;         // rows per wave
  static constexpr int WNR = BN / WN;         // LDS n-rows per wave
  static constexpr int MI = WMR / 32, NI = WNR / 32;
  static constexpr int A_CHUNKS = BM * 8 / NT;          // 16-B chunks per thread, K-contig A
  static constexpr int B_CHUNKS = BN * 8 / NT;
  static constexpr int A_UNITS = BM * 2 / NT;           // 4x8 transposed units per thread
  static constexpr int B_UNITS = BN * 2 / NT;
  static_assert(BM * 8 % NT == 0 && BN * 8 % NT == 0, "chunk split");
  static_assert(BM * 2 % NT == 0 && BN * 2 % NT == 0, "unit split");
  static_assert(WMR % 32 == 0 && WNR % 64 == 0, "wave tile");
};

// LDS n-row r of a tile -> (matrix, output column offset) of the op. Dual ops
// give each wave WNR/2 gate columns followed by the same WNR/2 up columns, so
// the gate and up accumulators of one output element share a lane.
template <class C, bool DUAL> MOE_DEV void nrow_map(int r, int& mat, int& col) {
  if (DUAL) {
    const int wn = r / C::WNR, w = r % C::WNR;
    mat = w / (C::WNR / 2);
    col = wn * (C::WNR / 2) + w % (C::WNR / 2);
  } else {
    mat = 0;
    col = r;
  }
}

template <int OP, class C>
__global__ void __launch_bounds__(C::NT, 1) gg_mfma_kernel(GGArgs a) {
  using I = OpInfo<OP>;
  constexpr bool DUAL = I::kDual, KVAR = I::kKVar, AK = I::kAKContig, BKC = I::kBKContig;
  constexpr int BM = C::BM, BN = C::BN, NT = C::NT, MI = C::MI, NI = C::NI;
  constexpr int BNO = DUAL ? BN / 2 : BN;   // output columns per matrix per tile
  __shared__ int tile_start[MOE_MAX_EXPERTS + 1];
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * kBK];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][BN * kBK];

  const int d = a.d, F = a.F;
  const int N = op_n(OP, d, F);
  const int tilesN = N / BNO;
  int e, row0, mv, K, m0 = 0, tn;
  if (!KVAR) {
    const int b = xcd_tile(blockIdx.x, gridDim.x, build_tile_prefix<BM, NT>(a, tile_start) * tilesN);
    if (b < 0) return;
    tn = b % tilesN;
    if (!m_tile_of<BM>(a, b / tilesN, tile_start, e, row0, mv)) return;
    K = op_k(OP, d, F);
  } else {
    const int b = xcd_remap(blockIdx.x, gridDim.x);
    const int M = op_wgrad_m(OP, d, F);
    const int per = (M / BM) * tilesN;
    e = b / per;
    m0 = ((b % per) / tilesN) * BM;
    tn = b % tilesN;
    group_rows(a, e, row0, K);
    mv = BM;
  }
  const int n0 = tn * BNO;
  const size_t dF = (size_t)d * F;
  const uint16_t* Ab = nullptr;        // A at (row 0 or m0, k 0)
  const uint16_t* Ab2 = nullptr;       // second K phase of DGRAD_GATE_UP
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
      Ab2 = (const uint16_t*)a.du + (size_t)row0 * F;
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

  const int tid = threadIdx.x;
  constexpr int RA = AK ? C::A_CHUNKS : 4 * C::A_UNITS;
  constexpr int RB = BKC ? C::B_CHUNKS : 4 * C::B_UNITS;
  V16 ra[RA], rb[RB];

  // ---- global -> registers
  auto load = [&](int k0) {
    if (AK) {
      const uint16_t* A = Ab;
      int kc0 = k0;
      if (OP == MOE_GG_DGRAD_GATE_UP && k0 >= F) { A = Ab2; kc0 = k0 - F; }
#pragma unroll
      for (int i = 0; i < C::A_CHUNKS; ++i) {
        const int q = i * NT + tid, m = q >> 3, kc = q & 7;
        ra[i] = m < mv ? *reinterpret_cast<const V16*>(A + (size_t)m * lda + kc0 + kc * 8) : zero16();
      }
    } else {
#pragma unroll
      for (int i = 0; i < C::A_UNITS; ++i) {
        const int u = i * NT + tid, o = u % (BM / 8), kq = u / (BM / 8);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int kk = k0 + 4 * kq + ii;
          ra[4 * i + ii] = kk < K ? *reinterpret_cast<const V16*>(Ab + (size_t)kk * lda + 8 * o) : zero16();
        }
      }
    }
    if (BKC) {
      const uint16_t* B = Bb[0];
      int kc0 = k0;
      if (OP == MOE_GG_DGRAD_GATE_UP && k0 >= F) { B = Bb[1]; kc0 = k0 - F; }
#pragma unroll
      for (int i = 0; i < C::B_CHUNKS; ++i) {
        const int q = i * NT + tid, n = q >> 3, kc = q & 7;
        rb[i] = *reinterpret_cast<const V16*>(B + (size_t)n * ldb + kc0 + kc * 8);
      }
    } else {
#pragma unroll
      for (int i = 0; i < C::B_UNITS; ++i) {
        const int u = i * NT + tid, o = u % (BN / 8), kq = u / (BN / 8);
        int mat, col;
        nrow_map<C, DUAL>(8 * o, mat, col);
        const uint16_t* B = Bb[mat];
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int kk = k0 + 4 * kq + ii;
          const bool ok = !KVAR || kk < K;
          rb[4 * i + ii] = ok ? *reinterpret_cast<const V16*>(B + (size_t)kk * ldb + col) : zero16();
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
      for (int i = 0; i < C::A_CHUNKS; ++i) {
        const int q = i * NT + tid, m = q >> 3, kc = q & 7;
        *reinterpret_cast<V16*>(A + lds_off(m, kc)) = ra[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < C::A_UNITS; ++i) {
        const int u = i * NT + tid, o = u % (BM / 8), kq = u / (BM / 8);
        store_transposed(A, 8 * o, kq, ra + 4 * i);
      }
    }
    if (BKC) {
#pragma unroll
      for (int i = 0; i < C::B_CHUNKS; ++i) {
        const int q = i * NT + tid, n = q >> 3, kc = q & 7;
        *reinterpret_cast<V16*>(B + lds_off(n, kc)) = rb[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < C::B_UNITS; ++i) {
        const int u = i * NT + tid, o = u % (BN / 8), kq = u / (BN / 8);
        store_transposed(B, 8 * o, kq, rb + 4 * i);
      }
    }
  };

  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int lr = lane & 31, lk = lane >> 5;
  // waves whose rows all lie past the tile's valid rows skip the matrix work
  const bool active = wm * C::WMR < mv;
  f32x16_t acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j)
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
    if (active) {
      const uint16_t* A = sA[cur];
      const uint16_t* B = sB[cur];
#pragma unroll
      for (int kk = 0; kk < kBK / 16; ++kk) {
        bf16x8_t af[MI], bfr[NI];
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
          af[mi] = *reinterpret_cast<const bf16x8_t*>(A + lds_off(wm * C::WMR + mi * 32 + lr, 2 * kk + lk));
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          bfr[ni] = *reinterpret_cast<const bf16x8_t*>(B + lds_off(wn * C::WNR + ni * 32 + lr, 2 * kk + lk));
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
          for (int ni = 0; ni < NI; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[ni], af[mi], acc[mi][ni], 0, 0, 0);
      }
    }
    if (kt + 1 < nk) store(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue. The MFMA ran with the B fragment first, so each 32x32
  // block holds C^T: lane (lr, lk) has output row lr and, for accumulator
  // group g, the 4 consecutive output columns 8g + 4lk .. 8g + 4lk + 3.
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
    const int ml = wm * C::WMR + mi * 32 + lr;
    if (ml >= mv) continue;
    const size_t row = KVAR ? (size_t)(m0 + ml) : (size_t)(row0 + ml);
#pragma unroll
    for (int ni = 0; ni < (DUAL ? NI / 2 : NI); ++ni) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int cl = ni * 32 + 8 * g + 4 * lk;
        float v0[4], v1[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          v0[r] = acc[mi][ni][4 * g + r];
          v1[r] = DUAL ? acc[mi][ni + NI / 2][4 * g + r] : 0.f;
        }
        if (OP == MOE_GG_FWD_GATE_UP) {
          const size_t i = row * F + n0 + wn * (C::WNR / 2) + cl;
          float gg[4], uu[4], hh[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            gg[r] = bf16_to_f32(f32_to_bf16(v0[r]));
            uu[r] = bf16_to_f32(f32_to_bf16(v1[r]));
            hh[r] = gg[r] * uu[r] / (1.0f + expf(-gg[r]));
          }
          *reinterpret_cast<uint2*>((uint16_t*)a.g + i) = pack4(gg);
          *reinterpret_cast<uint2*>((uint16_t*)a.u + i) = pack4(uu);
          *reinterpret_cast<uint2*>((uint16_t*)a.h + i) = pack4(hh);
        } else if (OP == MOE_GG_WGRAD_GATE_UP) {
          const size_t i = e * dF + row * F + n0 + wn * (C::WNR / 2) + cl;
          *reinterpret_cast<uint2*>((uint16_t*)a.dw_gate + i) = pack4(v0);
          *reinterpret_cast<uint2*>((uint16_t*)a.dw_up + i) = pack4(v1);
        } else if (OP == MOE_GG_DGRAD_DOWN) {
          const size_t i = row * F + n0 + wn * C::WNR + cl;
          float gf[4], uf[4], dg[4], du[4];
          unpack4(*reinterpret_cast<const uint2*>((const uint16_t*)a.g + i), gf);
          unpack4(*reinterpret_cast<const uint2*>((const uint16_t*)a.u + i), uf);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float s = 1.0f / (1.0f + expf(-gf[r]));
            dg[r] = v0[r] * uf[r] * s * (1.0f + gf[r] * (1.0f - s));
            du[r] = v0[r] * gf[r] * s;
          }
          *reinterpret_cast<uint2*>((uint16_t*)a.dg + i) = pack4(dg);
          *reinterpret_cast<uint2*>((uint16_t*)a.du + i) = pack4(du);
        } else {
          uint16_t* out;
          size_t i;
          if (OP == MOE_GG_FWD_DOWN) { out = (uint16_t*)a.y_perm; i = row * d; }
          else if (OP == MOE_GG_DGRAD_GATE_UP) { out = (uint16_t*)a.dx_perm; i = row * d; }
          else { out = (uint16_t*)a.dw_down; i = e * dF + row * d; }
          i += n0 + wn * C::WNR + cl;
          *reinterpret_cast<uint2*>(out + i) = pack4(v0);
        }
      }
    }
  }
}

}  // namespace moe
