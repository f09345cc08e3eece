// MXFP8 grouped expert GEMMs (gfx950): C ABI entry and launch. The pages
// credit MXFP8 for most of the feed-forward speed-up (bigchange.ai pt-BR,
// "Três números, três denominadores"); the kernel is in gemm_mx.h.
#include "gemm_mx.h"


namespace moe {
namespace {

// 128 x 256 tiles, a 3-deep ring, two workgroups per CU, 8 waves of 64 x 64.
using CfgMx = MxCfg<128, 256, 2, 4, 3, 2>;

template <int OP> void launch_mx_op(const MxArgs& x, int grid, hipStream_t s) {
  gg_mx_kernel<OP, CfgMx><<<grid, CfgMx::NT, 0, s>>>(x);
}

template <int OP> void launch_mx_split(const MxArgs& x, int grid, int* ws, hipStream_t s) {
  gg_mx_wgrad_split_kernel<OP, CfgMx><<<1, 256, 0, s>>>(x.o, grid, ws);
}

int launch_mx(int op, const MxArgs& x, int grid, hipStream_t s) {
  if (op == MOE_GG_WGRAD_DOWN || op == MOE_GG_WGRAD_GATE_UP) {
    int* ws = const_cast<int*>(x.o.split);
    if (op == MOE_GG_WGRAD_DOWN) launch_mx_split<MOE_GG_WGRAD_DOWN>(x, grid, ws, s);
    else launch_mx_split<MOE_GG_WGRAD_GATE_UP>(x, grid, ws, s);
    if (int st = launch_status()) return st;
  }
  switch (op) {
    case MOE_GG_FWD_GATE_UP: launch_mx_op<MOE_GG_FWD_GATE_UP>(x, grid, s); break;
    case MOE_GG_FWD_DOWN: launch_mx_op<MOE_GG_FWD_DOWN>(x, grid, s); break;
    case MOE_GG_DGRAD_DOWN: launch_mx_op<MOE_GG_DGRAD_DOWN>(x, grid, s); break;
    case MOE_GG_DGRAD_GATE_UP: launch_mx_op<MOE_GG_DGRAD_GATE_UP>(x, grid, s); break;
    case MOE_GG_WGRAD_DOWN: launch_mx_op<MOE_GG_WGRAD_DOWN>(x, grid, s); break;
    default: launch_mx_op<MOE_GG_WGRAD_GATE_UP>(x, grid, s); break;
  }
  return launch_status();
}

bool tensor_ok(const moe_mx_tensor& t) { return t.q != nullptr && t.s != nullptr && aligned16(t.q) && aligned4(t.s); }

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" size_t moe_grouped_gemm_mx_workspace_bytes(const moe_mx_gg_desc* desc) {
  if (desc == nullptr) return 0;
  const bool kvar = desc->op == MOE_GG_WGRAD_DOWN || desc->op == MOE_GG_WGRAD_GATE_UP;
  const int E = desc->E > 0 ? desc->E : 0;
  return kvar ? sizeof(int) * (size_t)(kMxColStart + E) : 0;
}

extern "C" int moe_grouped_gemm_mx(const moe_mx_gg_desc* g, hipStream_t stream) {
  MOE_CHECK_ARG(g != nullptr);
  MOE_CHECK_ARG(g->op >= MOE_GG_FWD_GATE_UP && g->op <= MOE_GG_WGRAD_GATE_UP);
  MOE_CHECK_ARG(g->E >= 1 && g->d > 0 && g->F > 0 && g->n_rows >= 0 && g->group_offsets != nullptr);
  MOE_CHECK_SUPPORTED(g->E <= MOE_MAX_EXPERTS && g->d % 256 == 0 && g->F % 256 == 0);
  const bool kvar = g->op == MOE_GG_WGRAD_DOWN || g->op == MOE_GG_WGRAD_GATE_UP;
  if (g->n_rows == 0 && !kvar) return MOE_OK;
  const long d = g->d, F = g->F, E = g->E;
  const bool rows = g->n_rows > 0;
  auto out_ok = [](const void* p) { return p != nullptr && aligned16(p); };
  // 32-bit buffer offsets: every operand's span from its expert base < 2 GiB
  long span = (long)g->n_rows * (d > F ? d : F);
  // MXFP8 copies written by the epilogue: H (FWD_GATE_UP) or dG and dU
  // (DGRAD_DOWN), each in both orientations, all given or none
  auto set = [](const moe_mx_tensor& t) { return t.q != nullptr || t.s != nullptr; };
  const bool qo = set(g->qo0_rows) || set(g->qo0_cols) || set(g->qo1_rows) || set(g->qo1_cols);
  switch (g->op) {
    case MOE_GG_FWD_GATE_UP:
      MOE_CHECK_ARG(tensor_ok(g->a0) && tensor_ok(g->b0) && tensor_ok(g->b1));
      // H in bf16 may be left out when its MXFP8 copies are written
      MOE_CHECK_ARG(out_ok(g->out0) && out_ok(g->out1) && (out_ok(g->out2) || (qo && g->out2 == nullptr)));
      span = span > F * E * d ? span : F * E * d;
      break;
    case MOE_GG_FWD_DOWN:
      MOE_CHECK_ARG(tensor_ok(g->a0) && tensor_ok(g->b0) && out_ok(g->out0));
      span = span > F * E * d ? span : F * E * d;
      break;
    case MOE_GG_DGRAD_DOWN:
      // dG and dU in bf16 may be left out (both) when their MXFP8 copies are written
      MOE_CHECK_ARG(tensor_ok(g->a0) && tensor_ok(g->b0));
      MOE_CHECK_ARG((out_ok(g->out0) && out_ok(g->out1)) || (qo && g->out0 == nullptr && g->out1 == nullptr));
      MOE_CHECK_ARG(out_ok(g->g) && out_ok(g->u));
      break;
    case MOE_GG_DGRAD_GATE_UP:
      MOE_CHECK_ARG(tensor_ok(g->a0) && tensor_ok(g->a1) && tensor_ok(g->b0) && tensor_ok(g->b1));
      MOE_CHECK_ARG(out_ok(g->out0));
      break;
    case MOE_GG_WGRAD_DOWN:
      MOE_CHECK_ARG(!rows || (tensor_ok(g->a0) && tensor_ok(g->b0)));
      MOE_CHECK_ARG(out_ok(g->out0));
      break;
    default:
      MOE_CHECK_ARG(!rows || (tensor_ok(g->a0) && tensor_ok(g->b0) && tensor_ok(g->b1)));
      MOE_CHECK_ARG(out_ok(g->out0) && out_ok(g->out1));
  }
  const int n_qo = (g->op == MOE_GG_FWD_GATE_UP) ? 1 : (g->op == MOE_GG_DGRAD_DOWN ? 2 : 0);
  if (qo) {
    MOE_CHECK_ARG(n_qo > 0);
    MOE_CHECK_ARG(tensor_ok(g->qo0_rows) && tensor_ok(g->qo0_cols));
    if (n_qo == 2) MOE_CHECK_ARG(tensor_ok(g->qo1_rows) && tensor_ok(g->qo1_cols));
    else MOE_CHECK_ARG(!set(g->qo1_rows) && !set(g->qo1_cols));
  }
  if (kvar || qo) {
    MOE_CHECK_ARG(g->col_stride > 0 && g->col_stride % 128 == 0);
    MOE_CHECK_ARG(g->col_stride >= 128L * ((g->n_rows + 127L) / 128 + E));
    const long cs = (long)(d > F ? d : F) * g->col_stride;
    span = span > cs ? span : cs;
  }
  MOE_CHECK_SUPPORTED(span < (1L << 31) && d * F < (1L << 31));
  const size_t ws_need = moe_grouped_gemm_mx_workspace_bytes(g);
  if (ws_need > 0 && (g->ws == nullptr || g->ws_bytes < ws_need || !aligned4(g->ws))) return MOE_ERR_WORKSPACE;

  MxArgs x{};
  x.o = GGArgs{g->op, g->E, g->d, g->F, g->n_rows, 0, g->group_offsets,
               nullptr, const_cast<void*>(g->g), const_cast<void*>(g->u), nullptr, nullptr, nullptr,
               nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
  switch (g->op) {
    case MOE_GG_FWD_GATE_UP: x.o.g = g->out0; x.o.u = g->out1; x.o.h = g->out2; break;
    case MOE_GG_FWD_DOWN: x.o.y_perm = g->out0; break;
    case MOE_GG_DGRAD_DOWN: x.o.dg = g->out0; x.o.du = g->out1; break;
    case MOE_GG_DGRAD_GATE_UP: x.o.dx_perm = g->out0; break;
    case MOE_GG_WGRAD_DOWN: x.o.dw_down = g->out0; break;
    default: x.o.dw_gate = g->out0; x.o.dw_up = g->out1;
  }
  auto put = [](const moe_mx_tensor& t, const uint8_t*& q, const uint8_t*& s) {
    q = static_cast<const uint8_t*>(t.q);
    s = static_cast<const uint8_t*>(t.s);
  };
  put(g->a0, x.aq[0], x.as[0]);
  put(g->a1, x.aq[1], x.as[1]);
  put(g->b0, x.bq[0], x.bs[0]);
  put(g->b1, x.bq[1], x.bs[1]);
  x.P = g->col_stride;
  x.o.split = ws_need > 0 ? static_cast<const int*>(g->ws) : nullptr;
  if (qo) {
    auto out = [](const moe_mx_tensor& r, const moe_mx_tensor& c) {
      return MxQOut{static_cast<uint8_t*>(const_cast<void*>(r.q)), static_cast<uint8_t*>(const_cast<void*>(r.s)),
                    static_cast<uint8_t*>(const_cast<void*>(c.q)), static_cast<uint8_t*>(const_cast<void*>(c.s))};
    };
    x.o.mxo[0] = out(g->qo0_rows, g->qo0_cols);
    if (n_qo == 2) x.o.mxo[1] = out(g->qo1_rows, g->qo1_cols);
    x.o.mx_P = g->col_stride;
  }

  const bool dual = g->op == MOE_GG_FWD_GATE_UP || g->op == MOE_GG_WGRAD_GATE_UP;
  const int N = op_n(g->op, g->d, g->F);
  const int bno = dual ? CfgMx::BN / 2 : CfgMx::BN;
  long grid;
  if (kvar) grid = E * (op_wgrad_m(g->op, g->d, g->F) / CfgMx::BM) * (N / bno);
  else grid = ((g->n_rows + CfgMx::BM - 1) / CfgMx::BM + E) * (long)(N / bno);
  MOE_CHECK_SUPPORTED(grid < (1L << 31));
  return launch_mx(g->op, x, static_cast<int>(grid), stream);
}
