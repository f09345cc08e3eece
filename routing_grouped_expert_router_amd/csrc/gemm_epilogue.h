// Output epilogue of the matrix-core grouped GEMMs: accumulators of a
// BM x BN tile -> bf16 outputs (with the SwiGLU forward or backward where the
// op has one), staged through LDS so that global traffic is whole 16-byte row
// segments.
#pragma once

#include "gemm_common.h"
#include "mx_common.h"

namespace moe {

typedef __attribute__((__vector_size__(16 * sizeof(float)))) float df32x16_t;

// sigmoid(x) = 1 / (1 + e^-x) with the hardware exponential and reciprocal
// (v_exp_f32 after the scaling by log2 e, v_rcp_f32): a few binary32 ulp from
// the correctly rounded value, far below the bf16 rounding of every output it
// feeds, and it takes the SwiGLU epilogues' VALU time off the GEMMs (an IEEE
// division is a dozen instructions). Large |x| give exactly 0 or 1.
MOE_DEV float fast_sigmoid(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

MOE_DEV uint2 dpack4(const float* v) { return make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])); }
MOE_DEV void dunpack4(uint2 p, float* v) {
  v[0] = __uint_as_float(p.x << 16);
  v[1] = __uint_as_float(p.x & 0xffff0000u);
  v[2] = __uint_as_float(p.y << 16);
  v[3] = __uint_as_float(p.y & 0xffff0000u);
}

// MXFP8 quantisation of one staged plane (BM rows x CW bf16 columns, row
// stride LDW) in both orientations, as moe_mx_quantize writes them with the
// experts as groups:
//  * rows: blocks of 32 along the columns; codes of the rows_valid valid rows
//    at q_rows[(grow0 + r) * K + col0 + ...], scale bytes in the grouped
//    layout of n_rows rows;
//  * cols: blocks of 32 along the tile's 128 rows (which start a 128-row
//    tile of the expert, so blocks restart at the expert's first row), the
//    rows past rows_valid counting as zeros; codes of output row col0 + c at
//    token column qcol0 + ..., scale bytes in the grouped layout of K rows.
// Each thread takes one 32-value block of each orientation per NT blocks,
// encoded from the staged bf16 words with the packed encoder (the codes the
// quantiser writes); scale bytes are stored one by one.
template <class C>
MOE_DEV void mx_quantize_plane(const uint16_t* stg, const MxQOut& o, size_t grow0, int rows_valid, int col0,
                               int K, int n_rows, int P, int qcol0, int tid) {
  constexpr int BM = C::BM, CW = C::CW, LDW = C::LDW, NT = C::NT;
  constexpr int RB = CW / 32, CB = BM / 32;        // blocks per tile row / per tile column
  for (int it = tid; it < BM * RB; it += NT) {
    const int r = it / RB, b = it % RB;
    uint32_t w[16];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const V16 t = *reinterpret_cast<const V16*>(stg + r * LDW + 32 * b + 8 * k);
#pragma unroll
      for (int m = 0; m < 4; ++m) w[4 * k + m] = t.w[m];
    }
    V16 out[2];
    const uint32_t code = quantize_block_bf16(w, out);
    if (r < rows_valid) {
      const size_t grow = grow0 + r;
      V16* qp = reinterpret_cast<V16*>(o.q_rows + grow * K + col0 + 32 * b);
      qp[0] = out[0];
      qp[1] = out[1];
      o.s_rows[4 * ((size_t)n_rows * (col0 / 128) + grow) + b] = static_cast<uint8_t>(code);
    }
  }
  for (int it = tid; it < CW * CB; it += NT) {
    const int c = it % CW, b = it / CW;
    uint32_t w[16];   // rows 2i, 2i+1 of the block in one word (rows past rows_valid: +0)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = 32 * b + 2 * i;
      const uint32_t lo = row < rows_valid ? stg[row * LDW + c] : 0u;
      const uint32_t hi = row + 1 < rows_valid ? stg[(row + 1) * LDW + c] : 0u;
      w[i] = lo | hi << 16;
    }
    V16 out[2];
    const uint32_t code = quantize_block_bf16(w, out);
    V16* qp = reinterpret_cast<V16*>(o.q_cols + (size_t)(col0 + c) * P + qcol0 + 32 * b);
    qp[0] = out[0];
    qp[1] = out[1];
    o.s_cols[4 * ((size_t)K * (qcol0 / 128) + col0 + c) + b] = static_cast<uint8_t>(code);
  }
}

// Each 32x32 block of acc holds C^T (B fragment first): lane (lr, lk) has
// tile row wm*WMR + mi*32 + lr and, for accumulator group g, the 4
// consecutive columns 8g + 4lk .. +3 of block ni. Output columns are handled
// in chunks of CW = 128 (one chunk per matrix for the dual ops, BN/128
// chunks otherwise); a wave's columns lie in one chunk. `lds` must hold
// 2 * BM * LDW bf16 values and be free for reuse (the caller's K loop is
// over: this function begins with a barrier). rbase is the first output row
// of the tile (permuted row, or weight row for the weight gradients) and n0
// its first output column; rows_valid rows are written.
// qcol0: token column of the tile's first row in the column orientation of
// the MXFP8 copies (the expert's first padded column plus the tile's first
// row within the expert), used when a.mxo is set.
// kchunk >= 0 (weight gradients with K split): the tile's binary32 sums over
// its K chunk go to a.partial as they are, straight from the accumulators
// (16-byte stores of four columns), for gg_splitk_reduce_kernel.
template <int OP, class C>
MOE_DEV void gg_store_tile(const GGArgs& a, const df32x16_t (&acc)[C::MI][C::NI], uint16_t* lds, int e,
                           size_t rbase, int n0, int rows_valid, int wm, int wn, int lane, int tid,
                           int qcol0 = 0, int kchunk = -1) {
  using I = OpInfo<OP>;
  constexpr bool DUAL = I::kDual;
  constexpr int MI = C::MI, NI = C::NI, NT = C::NT, BM = C::BM, BN = C::BN;
  constexpr int BNO = DUAL ? BN / 2 : BN;
  const int d = a.d, F = a.F;
  const size_t dF = (size_t)d * F;
  const int lr = lane & 31, lk = lane >> 5;
  constexpr int CW = C::CW, LDW = C::LDW;
  constexpr int NCH = BNO / CW > 0 ? BNO / CW : 1;          // column chunks per matrix
  constexpr int WCOLS = DUAL ? C::WNR / 2 : C::WNR;          // output columns per wave
  const int wcol0 = wn * WCOLS;                              // first output column of the wave
  const int wchunk = wcol0 / CW;
  uint16_t* stg0 = lds;
  uint16_t* stg1 = lds + BM * LDW;

  // value of accumulator element (mi, ni, g, r): tile row, chunk column
  auto row_of_acc = [&](int mi) { return wm * C::WMR + mi * 32 + lr; };
  auto col_of_acc = [&](int ni, int g) { return (wcol0 % CW) + ni * 32 + 8 * g + 4 * lk; };

  // cooperative copy of plane `src` (rows_valid x CW, columns chunk*CW..) to
  // global rows out + r * ld (+ chunk column offset)
  auto store_plane = [&](const uint16_t* src, uint16_t* out, size_t ld, int chunk) {
    constexpr int CPRW = CW / 8;                             // 16-byte chunks per row
    for (int q = tid; q < rows_valid * CPRW; q += NT) {
      const int r = q / CPRW, c = q % CPRW;
      *reinterpret_cast<V16*>(out + (size_t)r * ld + chunk * CW + c * 8) =
          *reinterpret_cast<const V16*>(src + r * LDW + c * 8);
    }
  };
  auto load_plane = [&](uint16_t* dst, const uint16_t* in, size_t ld, int chunk) {
    constexpr int CPRW = CW / 8;
    for (int q = tid; q < rows_valid * CPRW; q += NT) {
      const int r = q / CPRW, c = q % CPRW;
      *reinterpret_cast<V16*>(dst + r * LDW + c * 8) =
          *reinterpret_cast<const V16*>(in + (size_t)r * ld + chunk * CW + c * 8);
    }
  };
  // write 4 values as bf16 at (tile row, chunk column) of a staging plane
  auto put4 = [&](uint16_t* stg, int row, int col, const float* v) {
    *reinterpret_cast<uint2*>(stg + row * LDW + col) = dpack4(v);
  };

  if (I::kKVar && kchunk >= 0) {
    const int M = op_wgrad_m(OP, d, F), Nn = op_n(OP, d, F), NP = DUAL ? 2 * Nn : Nn;
    constexpr int NIH = DUAL ? NI / 2 : NI;   // column blocks per matrix
    float* base = a.partial + ((size_t)kchunk * a.E + e) * (size_t)M * NP;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const size_t row = rbase + row_of_acc(mi);
          const int col = (DUAL && ni >= NIH ? Nn : 0) + n0 + wcol0 + (ni % NIH) * 32 + 8 * g + 4 * lk;
          *reinterpret_cast<float4*>(base + row * NP + col) =
              make_float4(acc[mi][ni][4 * g], acc[mi][ni][4 * g + 1], acc[mi][ni][4 * g + 2], acc[mi][ni][4 * g + 3]);
        }
    return;
  }

  __syncthreads();   // every wave is done with the ring

  if (OP == MOE_GG_FWD_GATE_UP || OP == MOE_GG_WGRAD_GATE_UP) {
    // planes: G or dW_gate -> stg0, U or dW_up -> stg1
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI / 2; ++ni)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float v0[4], v1[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            v0[r] = acc[mi][ni][4 * g + r];
            v1[r] = acc[mi][ni + NI / 2][4 * g + r];
          }
          put4(stg0, row_of_acc(mi), col_of_acc(ni, g), v0);
          put4(stg1, row_of_acc(mi), col_of_acc(ni, g), v1);
        }
    __syncthreads();
    if (OP == MOE_GG_FWD_GATE_UP) {
      // G and U go out as staged; H = silu(g) * u from the same staged
      // (bf16-rounded) values, 8 per 16-byte chunk, written alongside
      constexpr int CPRW = CW / 8;
      uint16_t* outg = (uint16_t*)a.g + rbase * F + n0;
      uint16_t* outu = (uint16_t*)a.u + rbase * F + n0;
      uint16_t* outh = (uint16_t*)a.h + rbase * F + n0;
      const bool keep_gu = a.g != nullptr;   // null g and u: only h is written (recompute)
      const bool keep_h = a.h != nullptr;    // null h: H only as its MXFP8 copies
      for (int q = tid; q < rows_valid * CPRW; q += NT) {
        const int r = q / CPRW, c = q % CPRW;
        const V16 gv = *reinterpret_cast<const V16*>(stg0 + r * LDW + c * 8);
        const V16 uv = *reinterpret_cast<const V16*>(stg1 + r * LDW + c * 8);
        const size_t o = (size_t)r * F + c * 8;
        if (keep_gu) {
          *reinterpret_cast<V16*>(outg + o) = gv;
          *reinterpret_cast<V16*>(outu + o) = uv;
        }
        float gf[8], uf[8], hf[8];
        unpack(gv, gf);
        unpack(uv, uf);
#pragma unroll
        for (int i = 0; i < 8; ++i) hf[i] = gf[i] * uf[i] * fast_sigmoid(gf[i]);
        const V16 hv = pack(hf);
        if (keep_h) *reinterpret_cast<V16*>(outh + o) = hv;
        // H replaces G in the staging plane (this thread's chunk only) for
        // the MXFP8 copies below
        *reinterpret_cast<V16*>(stg0 + r * LDW + c * 8) = hv;
      }
      if (a.mxo[0].q_rows != nullptr) {
        __syncthreads();
        mx_quantize_plane<C>(stg0, a.mxo[0], rbase, rows_valid, n0, F, a.n_rows, a.mx_P, qcol0, tid);
      }
    } else {
      store_plane(stg0, (uint16_t*)a.dw_gate + e * dF + rbase * F + n0, F, 0);
      store_plane(stg1, (uint16_t*)a.dw_up + e * dF + rbase * F + n0, F, 0);
    }
  } else if (OP == MOE_GG_DGRAD_DOWN) {
    // per column chunk: stage G and U, turn them into dG and dU in place
    for (int ch = 0; ch < NCH; ++ch) {
      load_plane(stg0, (const uint16_t*)a.g + rbase * F + n0, F, ch);
      load_plane(stg1, (const uint16_t*)a.u + rbase * F + n0, F, ch);
      __syncthreads();
      if (wchunk == ch) {
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
          for (int ni = 0; ni < NI; ++ni)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int row = row_of_acc(mi), col = col_of_acc(ni, g);
              float gf[4], uf[4], dg[4], du[4];
              dunpack4(*reinterpret_cast<const uint2*>(stg0 + row * LDW + col), gf);
              dunpack4(*reinterpret_cast<const uint2*>(stg1 + row * LDW + col), uf);
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const float dh = acc[mi][ni][4 * g + r];
                const float sg = fast_sigmoid(gf[r]);
                dg[r] = dh * uf[r] * sg * (1.0f + gf[r] * (1.0f - sg));
                du[r] = dh * gf[r] * sg;
              }
              put4(stg0, row, col, dg);
              put4(stg1, row, col, du);
            }
      }
      __syncthreads();
      if (a.dg != nullptr) {   // null dg and du: dG and dU only as their MXFP8 copies
        store_plane(stg0, (uint16_t*)a.dg + rbase * F + n0, F, ch);
        store_plane(stg1, (uint16_t*)a.du + rbase * F + n0, F, ch);
      }
      if (a.mxo[0].q_rows != nullptr) {   // MXFP8 copies of this column chunk of dG and dU
        mx_quantize_plane<C>(stg0, a.mxo[0], rbase, rows_valid, n0 + ch * CW, F, a.n_rows, a.mx_P, qcol0, tid);
        mx_quantize_plane<C>(stg1, a.mxo[1], rbase, rows_valid, n0 + ch * CW, F, a.n_rows, a.mx_P, qcol0, tid);
      }
      __syncthreads();
    }
  } else {
    // single output: chunk 0 -> stg0, chunk 1 -> stg1 (at most two chunks)
    static_assert(NCH <= 2, "two staging planes");
    uint16_t* out;
    size_t ld;
    if (OP == MOE_GG_FWD_DOWN) { out = (uint16_t*)a.y_perm + rbase * d + n0; ld = d; }
    else if (OP == MOE_GG_DGRAD_GATE_UP) { out = (uint16_t*)a.dx_perm + rbase * d + n0; ld = d; }
    else { out = (uint16_t*)a.dw_down + e * dF + rbase * d + n0; ld = d; }
    uint16_t* mine = wchunk == 0 ? stg0 : stg1;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = acc[mi][ni][4 * g + r];
          put4(mine, row_of_acc(mi), col_of_acc(ni, g), v);
        }
    __syncthreads();
    store_plane(stg0, out, ld, 0);
    if (NCH > 1) store_plane(stg1, out, ld, 1);
  }
}

}  // namespace moe
