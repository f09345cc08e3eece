// bf16 grouped expert GEMM, matrix cores fed by direct global->LDS loads.
//
// One workgroup computes a BM x BN tile of one expert (BN counts LDS n-rows;
// for the dual ops half are gate columns and half are up columns). WM x WN
// wave64s each own a (BM/WM) x (BN/WN) sub-tile of 32 x 32 blocks of
// v_mfma_f32_32x32x16_bf16. K advances BK at a time through a ring of STAGES
// LDS buffers filled by buffer_load ... lds (16 bytes per lane, no register
// staging), so the loads of step k + STAGES - 1 are in flight while step k
// computes.
//
// Operand layouts in LDS:
//  * K-contiguous operands (rows of activations in the forward pass, weights
//    in dgrad) keep their rows: [rows][BK], 16-byte chunks XOR-swizzled by
//    (row >> 2) & 3 so that 16 consecutive rows of one chunk hit 16 distinct
//    bank groups; fragments are read with ds_read_b128.
//  * MN-contiguous operands (weights in the forward pass, everything in the
//    weight gradients) are copied as they are in memory: [BK][MN], 16-byte
//    chunks XOR-swizzled by 4 * (k & 3); fragments are read with two
//    ds_read_b64_tr_b16, whose 16-lane transpose turns four k-rows of four
//    columns into the k-contiguous fragment each lane needs.
// Tail rows (past an expert's rows, in M for the row-varying ops and in K for
// the weight gradients) read as zeros: every load goes through a buffer
// resource whose range ends at the expert's last row.
#pragma once

#include "gemm_epilogue.h"

namespace moe {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 dbf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short ds4_t;

template <int BM_, int BN_, int WM_, int WN_, int BK_, int ST_, int OCC_ = 1> struct DmaCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, BK = BK_, STAGES = ST_;
  static constexpr int OCC = OCC_;                         // workgroups per CU
  // waves per SIMD when OCC workgroups share a CU (HIP's second launch bound:
  // it caps the VGPRs per wave at 512 / this)
  static constexpr int WAVES_PER_SIMD = (WM_ * WN_ * OCC_ + 3) / 4;
  static constexpr int NT = WM * WN * 64;
  static constexpr int NW = WM * WN;
  static constexpr int WMR = BM / WM, WNR = BN / WN;
  static constexpr int MI = WMR / 32, NI = WNR / 32;
  static constexpr int CPR = BK / 8;                       // 16-byte chunks per K-contig row
  static constexpr int A_INSTR = BM * BK * 2 / 1024;       // 1 KB wave-loads per stage
  static constexpr int B_INSTR = BN * BK * 2 / 1024;
  static constexpr int A_PER_WAVE = A_INSTR / NW, B_PER_WAVE = B_INSTR / NW;
  static constexpr int STAGE_ELEMS = (BM + BN) * BK;
  // epilogue staging: two planes of BM rows x 128 columns (+8 padding)
  static constexpr int CW = 128, LDW = CW + 8;
  static constexpr int STAGING_ELEMS = 2 * BM * LDW;
  static constexpr int LDS_ELEMS = STAGE_ELEMS * STAGES > STAGING_ELEMS ? STAGE_ELEMS * STAGES : STAGING_ELEMS;
  static_assert(A_INSTR % NW == 0 && B_INSTR % NW == 0, "loads per wave");
  static_assert(BK == 32 || BK == 64, "K step");
  static_assert(WMR % 32 == 0 && WNR % 64 == 0, "wave tile");
  static_assert((BK * BN / 16) % 64 == 0, "dual sub-tiles hold whole wave-loads");
  // the MN-contiguous swizzle XORs chunk indices with up to 12: rows of an
  // MN-contiguous tile (A: BM, B: BN or BN/2 for the dual ops) need >= 16 chunks
  static_assert(BM >= 128 && BN / 2 >= 128, "MN-contiguous rows of >= 16 chunks");
  static_assert(OCC * (LDS_ELEMS * 2 + 4 * (MOE_MAX_EXPERTS + 1)) <= 160 * 1024, "LDS");
  static_assert(WNR <= CW && (BN <= CW || BN % CW == 0), "wave columns within one staging chunk");
};

// ------------------------------------------------------------------ primitives
// Raw buffer resource (4 SGPRs): 48-bit base, stride 0, range in bytes; loads
// past the range return zeros.
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int rsrc_t;
MOE_DEV rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  rsrc_t r;
  r[0] = __builtin_amdgcn_readfirstlane(static_cast<int>(p & 0xffffffffu));
  r[1] = __builtin_amdgcn_readfirstlane(static_cast<int>((p >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane(static_cast<int>(bytes));
  r[3] = 0x00020000;
  return r;
}

// One 1 KB wave-load: lane l's 16 bytes from byte offset voff of the resource
// land at LDS byte address lds_addr + 16 l. Issued from inline assembly so
// that the compiler, which cannot tell the ring slots apart, does not wait
// for every outstanding load before each LDS read; completion is tracked with
// explicit vmcnt waits instead (the instruction has no register result).
MOE_DEV void dma16(rsrc_t r, uint32_t lds_addr, uint32_t voff) {
  asm volatile(
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, 0 offen lds"
      :
      : "v"(voff), "s"(r), "{m0}"(lds_addr)
      : "memory");
}

MOE_DEV uint32_t lds_addr_of(const void* p) {
  typedef const __attribute__((address_space(3))) char* lds_ptr_t;
  return static_cast<uint32_t>((uintptr_t)(lds_ptr_t)p);
}

// s_waitcnt vmcnt(n) (expcnt and lgkmcnt left alone).
template <int N> MOE_DEV void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// chunk swizzles (16-byte chunk index within an LDS row)
MOE_DEV int swz_k(int row) { return (row >> 2) & 3; }      // K-contiguous rows
MOE_DEV int swz_t(int krow) { return (krow & 3) << 2; }     // MN-contiguous rows

MOE_DEV dbf16x8_t read_tr8(const uint16_t* p0, const uint16_t* p1) {
  const ds4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) ds4_t*)p0);
  const ds4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) ds4_t*)p1);
  typedef __attribute__((__vector_size__(8 * sizeof(short)))) short s8_t;
  const s8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(dbf16x8_t, v);
}

// ------------------------------------------------------------------ kernel
template <int OP, class C>
__global__ void __launch_bounds__(C::NT, C::WAVES_PER_SIMD) gg_dma_kernel(GGArgs a) {
  using I = OpInfo<OP>;
  constexpr bool DUAL = I::kDual, KVAR = I::kKVar, AK = I::kAKContig, BKC = I::kBKContig;
  constexpr int BM = C::BM, BN = C::BN, BK = C::BK, S = C::STAGES, NT = C::NT;
  constexpr int MI = C::MI, NI = C::NI, CPR = C::CPR;
  constexpr int BNO = DUAL ? BN / 2 : BN;          // output columns per matrix per tile
  constexpr int A_ELEMS = BM * BK;
  __shared__ int tile_start[MOE_MAX_EXPERTS + 1];
  __shared__ __attribute__((aligned(1024))) uint16_t lds[C::LDS_ELEMS];

  const int d = a.d, F = a.F;
  const int N = op_n(OP, d, F);
  const int tilesN = N / BNO;
  // one output tile: (expert, first row or weight row, valid rows, K, m0, n-tile)
  auto run_tile = [&](int e, int row0, int mv, int K, int m0, int tn, int kchunk = -1) {
    // the tile decode read LDS; its results are the same in every lane
    e = __builtin_amdgcn_readfirstlane(e);
    row0 = __builtin_amdgcn_readfirstlane(row0);
    mv = __builtin_amdgcn_readfirstlane(mv);
    K = __builtin_amdgcn_readfirstlane(K);
    m0 = __builtin_amdgcn_readfirstlane(m0);
    tn = __builtin_amdgcn_readfirstlane(tn);
    const int n0 = tn * BNO;
    const size_t dF = (size_t)d * F;

    // ---- buffer resources (byte ranges end at the last valid row)
    // A0/A1: the two K phases of DGRAD_GATE_UP (otherwise A1 = A0)
    // B0/B1: gate/up matrices (dual ops), or the two K phases (DGRAD_GATE_UP)
    rsrc_t rA0, rA1, rB0, rB1;
    int lda = 0, ldb = 0;
    {
      const uint16_t *pa0, *pa1, *pb0, *pb1;
      uint32_t na, nb;
      switch (OP) {
        case MOE_GG_FWD_GATE_UP:
          lda = d; ldb = F;
          pa0 = pa1 = (const uint16_t*)a.x_perm + (size_t)row0 * d; na = (uint32_t)mv * d * 2;
          pb0 = (const uint16_t*)a.w_gate + e * dF; pb1 = (const uint16_t*)a.w_up + e * dF; nb = (uint32_t)(dF * 2);
          break;
        case MOE_GG_FWD_DOWN:
          lda = F; ldb = d;
          pa0 = pa1 = (const uint16_t*)a.h + (size_t)row0 * F; na = (uint32_t)mv * F * 2;
          pb0 = pb1 = (const uint16_t*)a.w_down + e * dF; nb = (uint32_t)(dF * 2);
          break;
        case MOE_GG_DGRAD_DOWN:
          lda = d; ldb = d;
          pa0 = pa1 = (const uint16_t*)a.dy_perm + (size_t)row0 * d; na = (uint32_t)mv * d * 2;
          pb0 = pb1 = (const uint16_t*)a.w_down + e * dF; nb = (uint32_t)(dF * 2);
          break;
        case MOE_GG_DGRAD_GATE_UP:
          lda = F; ldb = F;
          pa0 = (const uint16_t*)a.dg + (size_t)row0 * F; pa1 = (const uint16_t*)a.du + (size_t)row0 * F;
          na = (uint32_t)mv * F * 2;
          pb0 = (const uint16_t*)a.w_gate + e * dF; pb1 = (const uint16_t*)a.w_up + e * dF; nb = (uint32_t)(dF * 2);
          break;
        case MOE_GG_WGRAD_DOWN:
          lda = F; ldb = d;
          pa0 = pa1 = (const uint16_t*)a.h + (size_t)row0 * F; na = (uint32_t)K * F * 2;
          pb0 = pb1 = (const uint16_t*)a.dy_perm + (size_t)row0 * d; nb = (uint32_t)K * d * 2;
          break;
        default:   // WGRAD_GATE_UP
          lda = d; ldb = F;
          pa0 = pa1 = (const uint16_t*)a.x_perm + (size_t)row0 * d; na = (uint32_t)K * d * 2;
          pb0 = (const uint16_t*)a.dg + (size_t)row0 * F; pb1 = (const uint16_t*)a.du + (size_t)row0 * F;
          nb = (uint32_t)K * F * 2;
      }
      rA0 = make_rsrc(pa0, na); rA1 = make_rsrc(pa1, na);
      rB0 = make_rsrc(pb0, nb); rB1 = make_rsrc(pb1, nb);
    }

    // the thread id passes through an empty asm so that the per-lane address
    // arithmetic below is redone for every tile of a weight-gradient
    // workgroup instead of being held in registers across its tile loop
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform

    // ---- per-lane byte offsets of this wave's loads at k = 0 (and their
    // increment per K step). A K-contiguous operand moves along its row; an
    // MN-contiguous one moves down BK rows.
    uint32_t a_off[C::A_PER_WAVE], b_off[C::B_PER_WAVE];
    int b_mat[C::B_PER_WAVE];
#pragma unroll
    for (int i = 0; i < C::A_PER_WAVE; ++i) {
      const int q = (wave * C::A_PER_WAVE + i) * 64 + lane;           // 16-byte chunk of the stage tile
      if (AK) {
        const int row = q / CPR, c = (q % CPR) ^ swz_k(row);
        a_off[i] = (uint32_t)(row * lda + c * 8) * 2;
      } else {   // [BK][BM]: BM/8 chunks per k-row
        const int kr = q / (BM / 8), c = (q % (BM / 8)) ^ swz_t(kr);
        a_off[i] = (uint32_t)(kr * lda + c * 8) * 2;
      }
    }
#pragma unroll
    for (int i = 0; i < C::B_PER_WAVE; ++i) {
      const int q = (wave * C::B_PER_WAVE + i) * 64 + lane;
      b_mat[i] = 0;
      if (BKC) {
        const int row = q / CPR, c = (q % CPR) ^ swz_k(row);
        b_off[i] = (uint32_t)((n0 + row) * ldb + c * 8) * 2;
      } else if (DUAL) {   // two [BK][BN/2] sub-tiles, gate then up
        // a 1 KB wave-load never straddles the sub-tiles, so the matrix is
        // wave-uniform and comes from the wave-load index alone
        const int sub = (wave * C::B_PER_WAVE + i) * 64 / (BK * BN / 16);
        const int qq = q % (BK * BN / 16);
        const int kr = qq / (BN / 16), c = (qq % (BN / 16)) ^ swz_t(kr);
        b_mat[i] = sub;
        b_off[i] = (uint32_t)(kr * ldb + n0 + c * 8) * 2;
      } else {
        const int kr = q / (BN / 8), c = (q % (BN / 8)) ^ swz_t(kr);
        b_off[i] = (uint32_t)(kr * ldb + n0 + c * 8) * 2;
      }
    }
    // wgrad A starts at column m0 of the token rows
    if (!AK) {
#pragma unroll
      for (int i = 0; i < C::A_PER_WAVE; ++i) a_off[i] += (uint32_t)m0 * 2;
    }
    const uint32_t a_step = AK ? BK * 2 : (uint32_t)BK * lda * 2;
    const uint32_t b_step = BKC ? BK * 2 : (uint32_t)BK * ldb * 2;

    // issue the loads of K step kt into ring slot `slot`
    const uint32_t lds_base = __builtin_amdgcn_readfirstlane(lds_addr_of(lds));
    // load i (A loads first, then B) of this wave's share of K step kt into
    // ring slot `slot`
    constexpr int PER_STAGE = C::A_PER_WAVE + C::B_PER_WAVE;   // wave-loads per stage
    auto issue_one = [&](int kt, int slot, int i) {
      const uint32_t sa = lds_base + (uint32_t)slot * C::STAGE_ELEMS * 2;
      const uint32_t sb = sa + A_ELEMS * 2;
      int ks = kt;
      bool second = false;
      if (OP == MOE_GG_DGRAD_GATE_UP) {
        const int half = F / BK;
        second = kt >= half;
        ks = second ? kt - half : kt;
      }
      if (i < C::A_PER_WAVE) {
        dma16(second ? rA1 : rA0, sa + (wave * C::A_PER_WAVE + i) * 1024, a_off[i] + (uint32_t)ks * a_step);
      } else {
        const int j = i - C::A_PER_WAVE;
        const bool use1 = DUAL ? (b_mat[j] != 0) : second;
        dma16(use1 ? rB1 : rB0, sb + (wave * C::B_PER_WAVE + j) * 1024, b_off[j] + (uint32_t)ks * b_step);
      }
    };
    auto issue = [&](int kt, int slot) {
#pragma unroll
      for (int i = 0; i < PER_STAGE; ++i) issue_one(kt, slot, i);
    };

    const int wm = wave / C::WN, wn = wave % C::WN;
    const int lr = lane & 31, lk = lane >> 5;
    // ds_read_b64_tr_b16 lane roles: 16-lane group g, source lane (j, q)
    const int tg = lane >> 4, tj = (lane & 15) >> 2, tq = lane & 3;
    const bool active = wm * C::WMR < mv;

    df32x16_t acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // fragments of K sub-step ks (16 deep) of ring slot `slot`
    auto read_frags = [&](int slot, int ks, dbf16x8_t (&af)[MI], dbf16x8_t (&bfr)[NI]) {
      const uint16_t* sa = lds + slot * C::STAGE_ELEMS;
      const uint16_t* sb = sa + A_ELEMS;
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        const int m = wm * C::WMR + mi * 32;
        if (AK) {
          const int row = m + lr;
          af[mi] = *reinterpret_cast<const dbf16x8_t*>(sa + row * BK + (((2 * ks + lk) ^ swz_k(row)) << 3));
        } else {
          const int col = m + 16 * (tg & 1) + 4 * tq;
          const int k0 = 16 * ks + 8 * (tg >> 1) + tj;
          const int k1 = k0 + 4;
          af[mi] = read_tr8(sa + k0 * BM + ((((col >> 3) ^ swz_t(k0)) << 3) | (col & 7)),
                            sa + k1 * BM + ((((col >> 3) ^ swz_t(k1)) << 3) | (col & 7)));
        }
      }
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        if (BKC) {
          const int row = wn * C::WNR + ni * 32 + lr;
          bfr[ni] = *reinterpret_cast<const dbf16x8_t*>(sb + row * BK + (((2 * ks + lk) ^ swz_k(row)) << 3));
        } else {
          const uint16_t* base = sb;
          int col, width;
          if (DUAL) {   // block ni < NI/2: gate sub-tile, else up sub-tile, same columns
            width = BN / 2;
            base = sb + (ni >= NI / 2 ? BK * (BN / 2) : 0);
            col = wn * (C::WNR / 2) + (ni % (NI / 2)) * 32;
          } else {
            width = BN;
            col = wn * C::WNR + ni * 32;
          }
          col += 16 * (tg & 1) + 4 * tq;
          const int k0 = 16 * ks + 8 * (tg >> 1) + tj;
          const int k1 = k0 + 4;
          bfr[ni] = read_tr8(base + k0 * width + ((((col >> 3) ^ swz_t(k0)) << 3) | (col & 7)),
                             base + k1 * width + ((((col >> 3) ^ swz_t(k1)) << 3) | (col & 7)));
        }
      }
    };
    auto mfmas = [&](const dbf16x8_t (&af)[MI], const dbf16x8_t (&bfr)[NI]) {
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[ni], af[mi], acc[mi][ni], 0, 0, 0);
    };

    // ---- K loop over a ring of S slots. Step kt has KS sub-steps of 16. The
    // fragments of each sub-step are read while the previous sub-step's MFMAs
    // run, so all of step kt's fragments are in registers before the barrier
    // that precedes its last sub-step (the barrier's fence drains LDS reads).
    // At that barrier every wave has waited for step kt+1; right after it the
    // slot of step kt is refilled with step kt+S, and step kt+1's first
    // fragments are read under step kt's last MFMAs. A step's loads thus have
    // S-1 steps to land.
    constexpr int KS = BK / 16;
    static_assert(S >= 2, "ring depth");
    const int nk = (K + BK - 1) / BK;
#pragma unroll
    for (int s = 0; s < S; ++s)
      if (s < nk) issue(s, s);
    dbf16x8_t af[2][MI], bfr[2][NI];
    // s_waitcnt vmcnt(PER_STAGE * n), n = stages allowed in flight (< S)
    auto wait_stages = [&](int n) {
      if (S > 3 && n >= 3) wait_vm<PER_STAGE * (S > 3 ? 3 : 0)>();
      else if (S > 2 && n == 2) wait_vm<PER_STAGE * (S > 2 ? 2 : 0)>();
      else if (n == 1) wait_vm<PER_STAGE>();
      else wait_vm<0>();
    };
    static_assert(S <= 4, "wait_stages covers up to three stages in flight");
    if (nk > 0) {
      wait_stages(min(S, nk) - 1);   // step 0 complete
      __syncthreads();
      if (active) read_frags(0, 0, af[0], bfr[0]);
    }
    for (int kt = 0; kt < nk; ++kt) {
      const int slot = kt % S;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int cur = ks & 1, nxt = cur ^ 1;
        if (ks + 1 < KS) {
          if (active) read_frags(slot, ks + 1, af[nxt], bfr[nxt]);
          if (active) mfmas(af[cur], bfr[cur]);
        } else {
          // steps issued so far end at min(kt + S - 1, nk - 1); step kt+1 must be complete
          if (kt + 1 < nk) wait_stages(min(kt + S - 1, nk - 1) - (kt + 1));
          __syncthreads();
          const bool refill = kt + S < nk;
          if (kt + 1 < nk && active) read_frags((kt + 1) % S, 0, af[nxt], bfr[nxt]);
          if (refill) issue(kt + S, slot);
          if (active) mfmas(af[cur], bfr[cur]);
        }
      }
    }

    gg_store_tile<OP, C>(a, acc, lds, e, KVAR ? (size_t)m0 : (size_t)row0, n0, mv, wm, wn, lane, tid, 0,
                         kchunk);
  };

  if constexpr (!KVAR) {
    int e, row0, mv, tn;
    const int b = xcd_tile(blockIdx.x, gridDim.x, build_tile_prefix<BM, NT>(a, tile_start) * tilesN);
    if (b < 0) return;
    // blocks of (expert's m-tiles) x (one n-tile): the m-tiles sharing a
    // weight slice run side by side (and fetch it from HBM once); experts are
    // visited in order
    if (!m_tile_grouped<BM>(a, b, tilesN, tile_start, e, row0, mv, tn)) return;
    run_tile(e, row0, mv, op_k(OP, d, F), 0, tn);
  } else if (a.ksplit > 1) {
    // K split: workgroup b takes chunk c of tile t, chunk-major (the tiles of
    // one chunk, which read the same rows, run side by side on an XCD); the
    // chunk is a run of whole K steps of the expert's rows
    const int tpe = (op_wgrad_m(OP, d, F) / BM) * tilesN;
    const int tiles = a.E * tpe;
    const int b = xcd_remap(blockIdx.x, gridDim.x);
    const int c = b / tiles, t = b % tiles;
    if (c >= a.ksplit) return;
    const int e = t / tpe;
    int row0, K;
    group_rows(a, e, row0, K);
    const int per = ((K + BK - 1) / BK + a.ksplit - 1) / a.ksplit * BK;
    const int k0 = min(K, c * per), k1 = min(K, k0 + per);
    run_tile(e, row0 + k0, BM, k1 - k0, ((t % tpe) / tilesN) * BM, t % tilesN, c);
  } else {
    const int tpe = (op_wgrad_m(OP, d, F) / BM) * tilesN;
    // The equal-count tile's group rows are fetched together with the split
    // flag, so a launch that does not balance waits on one load, not two.
    int t = xcd_remap(blockIdx.x, gridDim.x), end = t + 1, step = 1;
    int e = t / tpe, row0, K;
    group_rows(a, e, row0, K);
    if (a.split != nullptr && a.split[0] != 0) {
      wgrad_tiles(a.split, blockIdx.x, gridDim.x, t, end, step);
      if (t < end) {
        e = t / tpe;
        group_rows(a, e, row0, K);
      }
    }
    while (t < end) {
      run_tile(e, row0, BM, K, ((t % tpe) / tilesN) * BM, t % tilesN);
      t += step;
      if (t >= end) break;
      __syncthreads();   // the staging area is read to the end before the next tile's loads land
      e = t / tpe;
      group_rows(a, e, row0, K);
    }
  }
}

// Sum of the K chunks' binary32 partials of a split weight gradient, in
// chunk order (deterministic), rounded once to bf16: thread i takes the 8
// consecutive outputs 8i..8i+7 of the [E][M][NP] result.
template <int OP>
__global__ void __launch_bounds__(256) gg_splitk_reduce_kernel(GGArgs a) {
  constexpr bool DUAL = OpInfo<OP>::kDual;
  const int M = op_wgrad_m(OP, a.d, a.F), Nn = op_n(OP, a.d, a.F), NP = DUAL ? 2 * Nn : Nn;
  const size_t per = (size_t)a.E * M * NP;
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (i >= per) return;
  float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int c = 0; c < a.ksplit; ++c) {
    const float4* p = reinterpret_cast<const float4*>(a.partial + (size_t)c * per + i);
    const float4 v0 = p[0], v1 = p[1];
    s[0] += v0.x; s[1] += v0.y; s[2] += v0.z; s[3] += v0.w;
    s[4] += v1.x; s[5] += v1.y; s[6] += v1.z; s[7] += v1.w;
  }
  const size_t e = i / ((size_t)M * NP), rem = i % ((size_t)M * NP);
  const int m = (int)(rem / NP), n = (int)(rem % NP);
  const size_t dF = (size_t)a.d * a.F;
  uint16_t* out;
  if (OP == MOE_GG_WGRAD_DOWN) out = (uint16_t*)a.dw_down + e * dF + (size_t)m * Nn + n;
  else if (n < Nn) out = (uint16_t*)a.dw_gate + e * dF + (size_t)m * Nn + n;
  else out = (uint16_t*)a.dw_up + e * dF + (size_t)m * Nn + (n - Nn);
  *reinterpret_cast<V16*>(out) = pack(s);
}

// The tile split of one weight-gradient launch of nb workgroups (one
// workgroup; see wgrad_split).
template <int OP, class C>
__global__ void __launch_bounds__(256) gg_wgrad_split_kernel(GGArgs a, int nb, int* __restrict__ split) {
  __shared__ int scratch[MOE_MAX_EXPERTS + 1];
  constexpr int BNO = OpInfo<OP>::kDual ? C::BN / 2 : C::BN;
  const int tpe = (op_wgrad_m(OP, a.d, a.F) / C::BM) * (op_n(OP, a.d, a.F) / BNO);
  wgrad_split<C::BK, 256>(a, tpe, nb, scratch, split);
}

}  // namespace moe
