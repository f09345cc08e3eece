// MXFP8 grouped expert GEMM on the gfx950 scaled matrix cores.
//
// Every operand is E4M3 bytes plus one E8M0 scale byte per 32 values along the
// GEMM's contraction (K), stored with K contiguous, so each per-expert
// product is C[m][n] = sum_k A[m][k] B[n][k]. One v_mfma_scale_f32_32x32x64
// _f8f6f4 takes 64 K values of a 32-row block of each operand together with
// their scales and accumulates the exact scaled products in binary32.
//
// Operand layout of that instruction, for lane l of the wave (row l % 32 of
// the block, half h = l / 32): bytes 0..15 of its 32-byte operand are K values
// 16h..16h+15 of the first 32-block and bytes 16..31 are K values
// 32+16h..32+16h+15 of the second; the scale operand of lane l is the scale
// of row l % 32 in block h. Both operands use the same layout, so a row's 64
// bytes of one K step are read from LDS as two 16-byte chunks (h and 2 + h).
//
// The load path is the one of the bf16 kernel (gemm_dma.h): a ring of LDS
// stages filled with buffer_load ... lds. A stage holds 64 K values of the
// BM A-rows and BN B-rows (rows of 64 bytes, 16-byte chunks XOR-swizzled by
// (row >> 2) & 3) and one 4-byte word of scales per row: the scales of four
// 32-blocks, i.e. of this stage and the next (each word is loaded twice, by
// the two stages that use it, so every stage issues the same loads). The
// quantiser stores scale words of one 128-value column group contiguously
// over rows, so the words of 64 consecutive rows are one 256-byte load.
#pragma once

#include "gemm_dma.h"

namespace moe {

typedef __attribute__((__vector_size__(8 * sizeof(int)))) int di32x8_t;

// Workspace of the weight-gradient ops: the tile split, then from int
// kMxColStart one first padded token column per expert.
constexpr int kMxColStart = 16;
static_assert(kMxColStart >= kSplitInts, "split before the column starts");

struct MxArgs {
  GGArgs o;                 // shapes, group offsets, bf16 g/u inputs and the outputs
  const uint8_t* aq[2];     // A codes / scales (two K phases for DGRAD_GATE_UP)
  const uint8_t* as[2];
  const uint8_t* bq[2];     // B codes / scales (gate/up, or the two K phases)
  const uint8_t* bs[2];
  int P;                    // token stride of the column-quantised operands
};

template <int BM_, int BN_, int WM_, int WN_, int ST_, int OCC_> struct MxCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, STAGES = ST_, OCC = OCC_;
  // waves per SIMD when OCC workgroups share a CU (HIP's second launch bound)
  static constexpr int WAVES_PER_SIMD = (WM_ * WN_ * OCC_ + 3) / 4;
  static constexpr int BK = 64;                             // K values (bytes) per row per stage
  static constexpr int NT = WM * WN * 64, NW = WM * WN;
  static constexpr int WMR = BM / WM, WNR = BN / WN;
  static constexpr int MI = WMR / 32, NI = WNR / 32;
  static constexpr int A_PER_WAVE = BM * BK / 1024 / NW;    // 1 KB code wave-loads
  static constexpr int B_PER_WAVE = BN * BK / 1024 / NW;
  static constexpr int S_INSTR = (BM + BN) / 64;            // 256-byte scale wave-loads
  static constexpr int S_PER_WAVE = (S_INSTR + NW - 1) / NW;
  static constexpr int CODE_BYTES = (BM + BN) * BK;
  static constexpr int STAGE_BYTES = CODE_BYTES + (BM + BN) * 4;
  static constexpr int CW = 128, LDW = CW + 8;              // epilogue staging (bf16)
  static constexpr int STAGING_BYTES = 2 * BM * LDW * 2;
  static constexpr int RING_BYTES = STAGE_BYTES * STAGES;
  static constexpr int LDS_BYTES0 = RING_BYTES > STAGING_BYTES ? RING_BYTES : STAGING_BYTES;
  static constexpr int TS_BYTES = 4 * (MOE_MAX_EXPERTS + 1);
  static constexpr int LDS_BYTES = LDS_BYTES0 > TS_BYTES ? LDS_BYTES0 : TS_BYTES;
  static_assert(BM * BK % (1024 * NW) == 0 && BN * BK % (1024 * NW) == 0, "code loads per wave");
  static_assert(BM % 64 == 0 && BN % 128 == 0, "scale wave-loads stay within one operand and matrix");
  static_assert(WMR % 32 == 0 && WNR % 64 == 0, "wave tile");
  static_assert(STAGE_BYTES % 256 == 0, "stage alignment");
  static_assert(OCC * LDS_BYTES <= 160 * 1024, "LDS");
  static_assert(WNR <= CW && (BN <= CW || BN % CW == 0), "wave columns within one staging chunk");
  static_assert(STAGES >= 3, "ring depth");
};

// One 256-byte wave-load: lane l's 4 bytes land at LDS lds_addr + 4 l.
MOE_DEV void dma4(rsrc_t r, uint32_t lds_addr, uint32_t voff) {
  asm volatile(
      "s_nop 0\n\t"
      "buffer_load_dword %0, %1, 0 offen lds"
      :
      : "v"(voff), "s"(r), "{m0}"(lds_addr)
      : "memory");
}

// s_waitcnt vmcnt(PER * n) for a runtime n in [0, MAXN].
template <int PER, int MAXN> MOE_DEV void wait_stages(int n) {
  if constexpr (MAXN >= 2) {
    if (n >= 2) { wait_vm<PER * 2>(); return; }
  }
  if constexpr (MAXN >= 1) {
    if (n >= 1) { wait_vm<PER>(); return; }
  }
  wait_vm<0>();
}

template <int OP, class C>
__global__ void __launch_bounds__(C::NT, C::WAVES_PER_SIMD) gg_mx_kernel(MxArgs x) {
  using I = OpInfo<OP>;
  constexpr bool DUAL = I::kDual, KVAR = I::kKVar;
  constexpr int BM = C::BM, BN = C::BN, BK = C::BK, S = C::STAGES, NT = C::NT, NW = C::NW;
  constexpr int MI = C::MI, NI = C::NI;
  constexpr int BNO = DUAL ? BN / 2 : BN;          // output columns per matrix per tile
  static_assert(S - 2 <= 2, "wait_stages covers up to two stages in flight");
  static_assert(KVAR || BM == 128, "the MXFP8 copies' column tiles are the 128-row m-tiles");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[C::LDS_BYTES];
  int* tile_start = reinterpret_cast<int*>(lds);    // used before the ring, then overwritten

  const GGArgs& a = x.o;
  const int d = a.d, F = a.F, E = a.E;
  const int N = op_n(OP, d, F);
  const int tilesN = N / BNO;
  // one output tile: (expert, first row, valid rows, K, m0, n-tile, first
  // padded token column of the expert)
  auto run_tile = [&](int e, int row0, int mv, int K, int m0, int tn, int p_e) {
    // the tile decode read LDS or the workspace; its results are the same in every lane
    e = __builtin_amdgcn_readfirstlane(e);
    row0 = __builtin_amdgcn_readfirstlane(row0);
    mv = __builtin_amdgcn_readfirstlane(mv);
    K = __builtin_amdgcn_readfirstlane(K);
    m0 = __builtin_amdgcn_readfirstlane(m0);
    tn = __builtin_amdgcn_readfirstlane(tn);
    p_e = __builtin_amdgcn_readfirstlane(p_e);
    const int n0 = tn * BNO;
    // the thread id passes through an empty asm so that the per-lane address
    // arithmetic is redone for every tile of a weight-gradient workgroup
    // instead of being held in registers across its tile loop
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // ---- operands. Codes: base pointer of this expert's block (bytes), row
    // stride, range. Scales (grouped layout: the word of rows r, 128-value
    // column group c is at 4 * (R * c + r)): the whole buffer, its row count R,
    // the first column group g0 of this expert's K range, and the row of tile
    // row 0 (A: m, B: n before the dual split).
    const int P = x.P;
    const uint8_t *qa0, *qa1, *qb0, *qb1;
    uint32_t lda, ldb, na, nb;
    int sRa, sRb, g0a = 0, g0b = 0, rba, rbb;
    uint32_t sna, snb;
    switch (OP) {
      case MOE_GG_FWD_GATE_UP:
        lda = d; ldb = (uint32_t)E * d;
        qa0 = qa1 = x.aq[0] + (size_t)row0 * d; na = (uint32_t)mv * d;
        qb0 = x.bq[0] + (size_t)e * d; qb1 = x.bq[1] + (size_t)e * d;
        nb = (uint32_t)((size_t)F * E * d - (size_t)e * d);
        sRa = a.n_rows; rba = row0; sna = (uint32_t)a.n_rows * (d / 32);
        sRb = F; g0b = e * d / 128; rbb = n0; snb = (uint32_t)F * (E * d / 32);
        break;
      case MOE_GG_FWD_DOWN:
        lda = F; ldb = (uint32_t)E * F;
        qa0 = qa1 = x.aq[0] + (size_t)row0 * F; na = (uint32_t)mv * F;
        qb0 = qb1 = x.bq[0] + (size_t)e * F; nb = (uint32_t)((size_t)d * E * F - (size_t)e * F);
        sRa = a.n_rows; rba = row0; sna = (uint32_t)a.n_rows * (F / 32);
        sRb = d; g0b = e * F / 128; rbb = n0; snb = (uint32_t)d * (E * F / 32);
        break;
      case MOE_GG_DGRAD_DOWN:
        lda = d; ldb = d;
        qa0 = qa1 = x.aq[0] + (size_t)row0 * d; na = (uint32_t)mv * d;
        qb0 = qb1 = x.bq[0] + (size_t)e * F * d; nb = (uint32_t)F * d;
        sRa = a.n_rows; rba = row0; sna = (uint32_t)a.n_rows * (d / 32);
        sRb = E * F; rbb = e * F + n0; snb = (uint32_t)E * F * (d / 32);
        break;
      case MOE_GG_DGRAD_GATE_UP:
        lda = F; ldb = F;
        qa0 = x.aq[0] + (size_t)row0 * F; qa1 = x.aq[1] + (size_t)row0 * F; na = (uint32_t)mv * F;
        qb0 = x.bq[0] + (size_t)e * d * F; qb1 = x.bq[1] + (size_t)e * d * F; nb = (uint32_t)d * F;
        sRa = a.n_rows; rba = row0; sna = (uint32_t)a.n_rows * (F / 32);
        sRb = E * d; rbb = e * d + n0; snb = (uint32_t)E * d * (F / 32);
        break;
      case MOE_GG_WGRAD_DOWN:   // A = H^T [F][P], B = dY^T [d][P]
        lda = P; ldb = P;
        qa0 = qa1 = x.aq[0] + p_e; na = p_e < P ? (uint32_t)((size_t)F * P - p_e) : 0;
        qb0 = qb1 = x.bq[0] + p_e; nb = p_e < P ? (uint32_t)((size_t)d * P - p_e) : 0;
        sRa = F; g0a = p_e / 128; rba = m0; sna = (uint32_t)F * (P / 32);
        sRb = d; g0b = p_e / 128; rbb = n0; snb = (uint32_t)d * (P / 32);
        break;
      default:                  // WGRAD_GATE_UP: A = X^T [d][P], B = dG^T, dU^T [F][P]
        lda = P; ldb = P;
        qa0 = qa1 = x.aq[0] + p_e; na = p_e < P ? (uint32_t)((size_t)d * P - p_e) : 0;
        qb0 = x.bq[0] + p_e; qb1 = x.bq[1] + p_e; nb = p_e < P ? (uint32_t)((size_t)F * P - p_e) : 0;
        sRa = d; g0a = p_e / 128; rba = m0; sna = (uint32_t)d * (P / 32);
        sRb = F; g0b = p_e / 128; rbb = n0; snb = (uint32_t)F * (P / 32);
    }
    const rsrc_t rA0 = make_rsrc(qa0, na), rA1 = make_rsrc(qa1, na);
    const rsrc_t rB0 = make_rsrc(qb0, nb), rB1 = make_rsrc(qb1, nb);
    const rsrc_t rSA0 = make_rsrc(x.as[0], sna), rSA1 = make_rsrc(x.as[1] ? x.as[1] : x.as[0], sna);
    const rsrc_t rSB0 = make_rsrc(x.bs[0], snb), rSB1 = make_rsrc(x.bs[1] ? x.bs[1] : x.bs[0], snb);

    // ---- per-lane byte offsets at k = 0
    uint32_t a_off[C::A_PER_WAVE], b_off[C::B_PER_WAVE], s_off[C::S_PER_WAVE];
    int b_mat[C::B_PER_WAVE], s_kind[C::S_PER_WAVE], s_slot[C::S_PER_WAVE], s_R[C::S_PER_WAVE];
#pragma unroll
    for (int i = 0; i < C::A_PER_WAVE; ++i) {
      const int q = (wave * C::A_PER_WAVE + i) * 64 + lane;      // 16-byte chunk of the A stage tile
      const int row = q >> 2, c = (q & 3) ^ swz_k(row);
      a_off[i] = (uint32_t)(m0 + row) * lda + c * 16;
    }
#pragma unroll
    for (int i = 0; i < C::B_PER_WAVE; ++i) {
      const int q = (wave * C::B_PER_WAVE + i) * 64 + lane;
      const int row = q >> 2, c = (q & 3) ^ swz_k(row);
      // a 1 KB wave-load covers 16 rows, so the matrix is wave-uniform
      const int sub = DUAL ? ((wave * C::B_PER_WAVE + i) * 16) / (BN / 2) : 0;
      b_mat[i] = sub;
      b_off[i] = (uint32_t)(n0 + row - sub * (BN / 2)) * ldb + c * 16;
    }
#pragma unroll
    for (int i = 0; i < C::S_PER_WAVE; ++i) {
      int j = wave * C::S_PER_WAVE + i;
      if (j >= C::S_INSTR) j -= C::S_INSTR;   // spare loads repeat one of the others (same bytes, same place)
      s_slot[i] = j;
      const int srow = 64 * j + lane;         // rows: A 0..BM-1, then B
      if (64 * j < BM) {
        s_kind[i] = 0;
        s_R[i] = sRa;
        s_off[i] = 4u * ((uint32_t)g0a * sRa + rba + srow);
      } else {
        const int rb = srow - BM;
        const int sub = DUAL ? (64 * j - BM) / (BN / 2) : 0;
        s_kind[i] = 1 + sub;
        s_R[i] = sRb;
        s_off[i] = 4u * ((uint32_t)g0b * sRb + rbb + rb - sub * (BN / 2));
      }
    }

    const uint32_t lds_base = __builtin_amdgcn_readfirstlane(lds_addr_of(lds));
    // Resources are picked by branching on wave-uniform conditions rather than
    // by selecting between them, so that each load names one SGPR quad.
    auto issue_phase = [&](uint32_t sa, int ks, const rsrc_t& ra, const rsrc_t& rb, const rsrc_t& rsa,
                           const rsrc_t& rsb) {
      const uint32_t sb = sa + BM * BK;
      const uint32_t ss = sa + C::CODE_BYTES;
#pragma unroll
      for (int i = 0; i < C::A_PER_WAVE; ++i)
        dma16(ra, sa + (wave * C::A_PER_WAVE + i) * 1024, a_off[i] + (uint32_t)ks * BK);
#pragma unroll
      for (int i = 0; i < C::B_PER_WAVE; ++i) {
        const uint32_t dst = sb + (wave * C::B_PER_WAVE + i) * 1024, off = b_off[i] + (uint32_t)ks * BK;
        if (DUAL && b_mat[i] != 0) dma16(rB1, dst, off);
        else dma16(rb, dst, off);
      }
#pragma unroll
      for (int i = 0; i < C::S_PER_WAVE; ++i) {
        const uint32_t dst = ss + s_slot[i] * 256, off = s_off[i] + 4u * (uint32_t)(ks >> 1) * s_R[i];
        if (s_kind[i] == 0) dma4(rsa, dst, off);
        else if (DUAL && s_kind[i] == 2) dma4(rSB1, dst, off);
        else dma4(rsb, dst, off);
      }
    };
    auto issue = [&](int kt, int slot) {
      const uint32_t sa = lds_base + (uint32_t)slot * C::STAGE_BYTES;
      if (OP == MOE_GG_DGRAD_GATE_UP) {
        const int half = F / BK;
        if (kt >= half) issue_phase(sa, kt - half, rA1, rB1, rSA1, rSB1);
        else issue_phase(sa, kt, rA0, rB0, rSA0, rSB0);
      } else {
        issue_phase(sa, kt, rA0, rB0, rSA0, rSB0);
      }
    };

    const int wm = wave / C::WN, wn = wave % C::WN;
    const int lr = lane & 31, lk = lane >> 5;
    const bool active = wm * C::WMR < mv;

    df32x16_t acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // fragments and scale words of stage kt (ring slot `slot`)
    auto read_frags = [&](int slot, int kt, di32x8_t (&af)[MI], di32x8_t (&bfr)[NI], int (&sa)[MI], int (&sb)[NI]) {
      const uint8_t* st = lds + slot * C::STAGE_BYTES;
      const uint32_t* sw = reinterpret_cast<const uint32_t*>(st + C::CODE_BYTES);
      const int sh = 8 * (2 * (kt & 1) + lk);
      auto frag = [&](const uint8_t* base, int row) {
        const uint4 lo = *reinterpret_cast<const uint4*>(base + row * BK + ((lk ^ swz_k(row)) << 4));
        const uint4 hi = *reinterpret_cast<const uint4*>(base + row * BK + (((2 + lk) ^ swz_k(row)) << 4));
        const di32x8_t v = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        return v;
      };
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        const int row = wm * C::WMR + mi * 32 + lr;
        af[mi] = frag(st, row);
        sa[mi] = (int)(sw[row] >> sh);
      }
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        int row;
        if (DUAL) row = (ni >= NI / 2 ? BN / 2 : 0) + wn * (C::WNR / 2) + (ni % (NI / 2)) * 32 + lr;
        else row = wn * C::WNR + ni * 32 + lr;
        bfr[ni] = frag(st + BM * BK, row);
        sb[ni] = (int)(sw[BM + row] >> sh);
      }
    };
    auto mfmas = [&](const di32x8_t (&af)[MI], const di32x8_t (&bfr)[NI], const int (&sa)[MI], const int (&sb)[NI]) {
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bfr[ni], af[mi], acc[mi][ni], 0, 0, 0,
                                                                       sb[ni], 0, sa[mi]);
    };

    // ---- K loop: one MFMA depth per stage. At step kt every wave waits for
    // stage kt, meets the others at one barrier, refills the slot of stage
    // kt-1 (read and consumed by every wave before this barrier) with stage
    // kt+S-1, then reads stage kt's fragments and runs its MFMAs; the other
    // workgroup on the CU covers the fragment reads. Loads get S-1 steps to land.
    constexpr int PER_STAGE = C::A_PER_WAVE + C::B_PER_WAVE + C::S_PER_WAVE;
    int nk = (K + BK - 1) / BK;
    // an expert's token columns end inside the col_stride P (always so for
    // group offsets that keep the documented contract)
    if (KVAR) nk = p_e >= P ? 0 : min(nk, (P - p_e) / BK);
#pragma unroll
    for (int s = 0; s < S - 1; ++s)
      if (s < nk) issue(s, s);
    for (int kt = 0; kt < nk; ++kt) {
      // stages issued so far end at min(kt + S - 2, nk - 1); stage kt must be complete
      wait_stages<PER_STAGE, S - 2>(min(kt + S - 2, nk - 1) - kt);
      __syncthreads();
      if (kt + S - 1 < nk) issue(kt + S - 1, (kt + S - 1) % S);
      if (active) {
        di32x8_t af[MI], bfr[NI];
        int saw[MI], sbw[NI];
        read_frags(kt % S, kt, af, bfr, saw, sbw);
        mfmas(af, bfr, saw, sbw);
      }
    }

    // the row-varying ops receive in p_e the column-orientation token column
    // of their first row (for the MXFP8 copies the epilogue may write)
    gg_store_tile<OP, C>(a, acc, reinterpret_cast<uint16_t*>(lds), e, KVAR ? (size_t)m0 : (size_t)row0, n0, mv,
                         wm, wn, lane, tid, KVAR ? 0 : p_e);
  };

  if constexpr (!KVAR) {
    int e, row0, mv, tn;
    const int b = xcd_tile(blockIdx.x, gridDim.x, build_tile_prefix<BM, NT>(a, tile_start) * tilesN);
    if (b < 0) return;
    if (!m_tile_grouped<BM>(a, b, tilesN, tile_start, e, row0, mv, tn)) return;
    // token column of the tile's first row in the column orientation: the
    // expert's first padded column (128 per m-tile of the experts before it,
    // BM = 128) plus the row's offset within the expert
    int r0e, ne;
    group_rows(a, e, r0e, ne);
    const int qcol0 = 128 * tile_start[e] + (row0 - r0e);
    __syncthreads();   // every wave is past its reads of tile_start before the ring is filled
    run_tile(e, row0, mv, op_k(OP, d, F), 0, tn, qcol0);
  } else {
    // the workspace holds the launch's tile split (wgrad_tiles) and each
    // expert's first padded token column (gg_mx_wgrad_split_kernel)
    const int* __restrict__ ws = a.split;
    const int tpe = (op_wgrad_m(OP, d, F) / BM) * tilesN;
    // the equal-count tile's rows and column start are fetched together with
    // the split flag
    int t = xcd_remap(blockIdx.x, gridDim.x), end = t + 1, step = 1;
    int e = t / tpe, row0, K;
    group_rows(a, e, row0, K);
    int p_e = ws[kMxColStart + e];
    if (ws[0] != 0) {
      wgrad_tiles(ws, blockIdx.x, gridDim.x, t, end, step);
      if (t < end) {
        e = t / tpe;
        group_rows(a, e, row0, K);
        p_e = ws[kMxColStart + e];
      }
    }
    while (t < end) {
      run_tile(e, row0, BM, K, ((t % tpe) / tilesN) * BM, t % tilesN, p_e);
      t += step;
      if (t >= end) break;
      __syncthreads();   // the staging area is read to the end before the next tile's loads land
      e = t / tpe;
      group_rows(a, e, row0, K);
      p_e = ws[kMxColStart + e];
    }
  }
}

// One workgroup, before an MXFP8 weight-gradient launch of nb workgroups:
// the launch's tile split (ws[0, kSplitInts), see wgrad_split, with this
// kernel's K step) and each expert's first padded token column,
// ws[kMxColStart + e] = 128 * sum over h < e of ceil(rows of h / 128).
template <int OP, class C>
__global__ void __launch_bounds__(256) gg_mx_wgrad_split_kernel(GGArgs a, int nb, int* __restrict__ ws) {
  __shared__ int scratch[MOE_MAX_EXPERTS + 1];
  constexpr int BNO = OpInfo<OP>::kDual ? C::BN / 2 : C::BN;
  const int tpe = (op_wgrad_m(OP, a.d, a.F) / C::BM) * (op_n(OP, a.d, a.F) / BNO);
  wgrad_split<C::BK, 256>(a, tpe, nb, scratch, ws);
  __syncthreads();   // scratch is reused below
  build_expert_prefix<256>(a.E, [&](int e) {
    int r0, n;
    group_rows(a, e, r0, n);
    return (n + 127) >> 7;
  }, scratch);
  for (int e = threadIdx.x; e < a.E; e += 256) ws[kMxColStart + e] = 128 * scratch[e];
}

}  // namespace moe
