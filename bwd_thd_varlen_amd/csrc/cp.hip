// Merge of two partial attention results over disjoint key sets: the step
// that combines attention computed chunk by chunk over the keys (context
// parallelism keeps a sequence's keys in chunks; TransformerEngine issue
// 3333, section "What we ruled out", mentions it only in passing).
//
// With P_a = exp(S - LSE_a) on key set A (O_a = P_a V_A) and likewise for B,
// the softmax over A u B has LSE = ln(e^LSE_a + e^LSE_b) and
// O = e^(LSE_a - LSE) O_a + e^(LSE_b - LSE) O_b.  A side with LSE = -inf has
// weight 0; both empty give O = 0, LSE = -inf (padding rows stay as they are).
//
// In place on (out, lse).  CHP lanes (a power of two >= d/8) share one
// (row, head): they sit in one wave, whose single load instruction reads the
// old LSE for all of them before any lane stores the new one.
#include "common.h"

namespace attn {

struct MergeParams {
  void* out;
  float* lse;
  const void* out_part;
  const float* lse_part;
  int64_t rows;      // total_q * hq
  int32_t d;
};

template <int DT, int CHP>
__global__ __launch_bounds__(256) void merge_kernel(MergeParams p) {
  static_assert(CHP <= 64 && (64 % CHP) == 0, "a (row, head) stays inside one wave");
  constexpr int kRowsPerBlock = 256 / CHP;
  const int tid = threadIdx.x;
  const int c = tid & (CHP - 1);
  const int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + tid / CHP;
  if (r >= p.rows) return;
  const float la = p.lse[r], lb = p.lse_part[r];
  const float m = fmaxf(la, lb);
  float wa = 0.f, wb = 0.f, l = -__builtin_inff();
  if (m != -__builtin_inff()) {
    const float ea = expf(la - m), eb = expf(lb - m);   // one of them is 1
    const float s = ea + eb;
    wa = ea / s;
    wb = eb / s;
    l = m + logf(s);
  }
  if (8 * c < p.d) {
    uint16_t* o = reinterpret_cast<uint16_t*>(p.out) + r * p.d + 8 * c;
    const u32x4 a = *reinterpret_cast<const u32x4*>(o);
    const u32x4 b = ldg16(reinterpret_cast<const uint16_t*>(p.out_part) + r * p.d + 8 * c);
    u32x4 res;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t aw = a[w], bw = b[w];
      const f32x2 x = Mfma<DT>::unpack2(aw), y = Mfma<DT>::unpack2(bw);
      res[w] = Mfma<DT>::pack2(wa * x[0] + wb * y[0], wa * x[1] + wb * y[1]);
    }
    *reinterpret_cast<u32x4*>(o) = res;
  }
  if (c == 0) p.lse[r] = l;
}

template <int DT>
static void launch_merge_dt(const MergeParams& p, hipStream_t st) {
  const int ch = p.d >> 3;
  auto grid = [&](int chp) { return (unsigned)((p.rows + 256 / chp - 1) / (256 / chp)); };
  if (ch <= 1) hipLaunchKernelGGL((merge_kernel<DT, 1>), dim3(grid(1)), dim3(256), 0, st, p);
  else if (ch <= 2) hipLaunchKernelGGL((merge_kernel<DT, 2>), dim3(grid(2)), dim3(256), 0, st, p);
  else if (ch <= 4) hipLaunchKernelGGL((merge_kernel<DT, 4>), dim3(grid(4)), dim3(256), 0, st, p);
  else if (ch <= 8) hipLaunchKernelGGL((merge_kernel<DT, 8>), dim3(grid(8)), dim3(256), 0, st, p);
  else if (ch <= 16) hipLaunchKernelGGL((merge_kernel<DT, 16>), dim3(grid(16)), dim3(256), 0, st, p);
  else hipLaunchKernelGGL((merge_kernel<DT, 32>), dim3(grid(32)), dim3(256), 0, st, p);
}

hipError_t launch_merge(void* out, float* lse, const void* out_part, const float* lse_part,
                        int64_t rows, int d, int dtype, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  MergeParams p{out, lse, out_part, lse_part, rows, d};
  if (dtype == kBF16) launch_merge_dt<kBF16>(p, st);
  else launch_merge_dt<kFP16>(p, st);
  return hipGetLastError();
}

}  // namespace attn
