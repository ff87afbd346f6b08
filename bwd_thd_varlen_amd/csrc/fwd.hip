// Forward kernel: O = softmax(scale * Q K^T + mask) V and LSE, per
// (sequence, 128-query tile, query head).
//
// TransformerEngine issue 3333 ("FusedAttention (cuDNN) THD backward ...",
// section "Reproduction") defines the result as a per-sequence SDPA; issue
// 3216 ("flash-attn-4 ...", section "Reproduce") fixes the GQA head map
// (query head h reads KV head h / (hq/hkv)) and the causal triangle.
//
// Work split: 4 waves x 32 queries.  Each lane owns one query (column of the
// transposed score tile S^T = K Q^T), so the softmax statistics are per-lane
// scalars and the probabilities, still in registers, are directly the B
// operand of O^T = V^T P^T.  Q stays in registers for the whole tile; each
// 64-key step stages K (row-major) and V^T (transposed, perm16 order) in LDS,
// the next step's K/V being fetched into registers while this one computes.
// Online softmax in the log2 domain: m = running max of scale*log2(e)*S,
// l = running sum of exp2(x - m), O rescaled by exp2(m_old - m_new) only when
// some lane's maximum moved.
#include "common.h"

namespace attn {

template <int DT, int DPAD, bool CAUSAL>
__global__ __launch_bounds__(256, DPAD <= 128 ? 2 : 1) void fwd_kernel(AttnParams p) {
  constexpr int NT = DPAD / 16;        // 16-wide k chunks over the head dim
  constexpr int NCB = DPAD / 32;       // 32-row blocks of O^T
  constexpr int KS = kKVStep;          // keys per step
  constexpr int SKS = DPAD + 8;        // K row stride in LDS (elements)
  constexpr int SVS = KS + 8;          // V^T row stride in LDS (elements)
  constexpr int CPR = DPAD / 8;        // 16-byte chunks per row
  constexpr int UNITS = (KS / 4) * CPR;
  constexpr int UPT = (UNITS + 255) / 256;

  __shared__ __attribute__((aligned(16))) uint16_t sK[KS * SKS];
  __shared__ __attribute__((aligned(16))) uint16_t sVt[DPAD * SVS];

  const int ntiles = p.hdr[kHdrNQTiles];
  int item, h;
  xcd_split(blockIdx.x, p.hq, item, h);
  if (item >= ntiles) return;
  const int2 e = p.list[item];
  const SeqInfo s = p.seq[e.x];
  const int g = h / p.group;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 31, hh = lane >> 5;
  const int m0 = e.y * kQTile;
  const int qi = m0 + wave * 32 + li;
  const int wq_lo = m0 + wave * 32, wq_hi = wq_lo + 31;
  const int64_t qrs = (int64_t)p.hq * p.d, kvrs = (int64_t)p.hkv * p.d;
  const uint16_t* qb = reinterpret_cast<const uint16_t*>(p.q) + (int64_t)s.oq * qrs + (int64_t)h * p.d;
  const uint16_t* kb = reinterpret_cast<const uint16_t*>(p.k) + (int64_t)s.ok * kvrs + (int64_t)g * p.d;
  const uint16_t* vb = reinterpret_cast<const uint16_t*>(p.v) + (int64_t)s.ok * kvrs + (int64_t)g * p.d;
  const u32x4 z4 = {0u, 0u, 0u, 0u};

  u32x4 qreg[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int c = 16 * t + 8 * hh;
    qreg[t] = (qi < s.lq && c < p.d) ? ldg16(qb + (int64_t)qi * qrs + c) : z4;
  }

  const int q_end = min(s.lq, m0 + kQTile);
  const int kend = CAUSAL ? min(s.lk, q_end) : s.lk;
  const int nsteps = (kend + KS - 1) / KS;
  const float sl2e = p.scale_log2e;

  f32x16 acc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) acc[cb] = zero16();
  float m_run = -__builtin_inff(), l_run = 0.f;

  u32x4 pk[UPT][4], pv[UPT][4];
  auto load_step = [&](int step) {
    const int n0 = step * KS;
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int unit = tid + 256 * u;
      const int rg = unit / CPR, cc = unit - rg * CPR;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = n0 + 4 * rg + r;
        const bool ok = unit < UNITS && j < kend && 8 * cc < p.d;
        const int64_t off = (int64_t)j * kvrs + 8 * cc;
        pk[u][r] = ok ? ldg16(kb + off) : z4;
        pv[u][r] = ok ? ldg16(vb + off) : z4;
      }
    }
  };
  auto store_step = [&]() {
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int unit = tid + 256 * u;
      if (UNITS % 256 != 0 && unit >= UNITS) continue;
      const int rg = unit / CPR, cc = unit - rg * CPR;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        *reinterpret_cast<u32x4*>(&sK[(4 * rg + r) * SKS + 8 * cc]) = pk[u][r];
      const int pos = perm16(4 * rg);
#pragma unroll
      for (int e8 = 0; e8 < 8; ++e8) {
        const int w = e8 >> 1, sh = (e8 & 1) * 16;
        const uint32_t x0 = (pv[u][0][w] >> sh) & 0xffffu, x1 = (pv[u][1][w] >> sh) & 0xffffu;
        const uint32_t x2 = (pv[u][2][w] >> sh) & 0xffffu, x3 = (pv[u][3][w] >> sh) & 0xffffu;
        u32x2 val = {x0 | (x1 << 16), x2 | (x3 << 16)};
        *reinterpret_cast<u32x2*>(&sVt[(8 * cc + e8) * SVS + pos]) = val;
      }
    }
  };

  if (nsteps > 0) load_step(0);
  for (int step = 0; step < nsteps; ++step) {
    __syncthreads();
    store_step();
    __syncthreads();
    if (step + 1 < nsteps) load_step(step + 1);
    const int n0 = step * KS;
    if (wq_lo >= s.lq) continue;                 // no real query in this wave
    if (CAUSAL && n0 > wq_hi) continue;          // whole step above this wave's diagonal

    f32x16 sc[2];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      sc[kb2] = zero16();
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(&sK[(32 * kb2 + li) * SKS + 16 * t + 8 * hh]);
        sc[kb2] = Mfma<DT>::mma(a, qreg[t], sc[kb2]);
      }
    }
    const bool need_mask = (n0 + KS > kend) || (CAUSAL && n0 + KS - 1 > wq_lo);
    if (need_mask) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = n0 + 32 * kb2 + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (j >= kend || (CAUSAL && j > qi)) sc[kb2][r] = -__builtin_inff();
        }
    }
    float mx = -__builtin_inff();
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kb2][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx * sl2e);
    const float base = (m_new == -__builtin_inff()) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - base);
    float rsum = 0.f;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pr = fast_exp2(__builtin_fmaf(sc[kb2][r], sl2e, -base));
        sc[kb2][r] = pr;
        rsum += pr;
      }
    l_run = l_run * alpha + rsum;
    m_run = m_new;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[cb][r] *= alpha;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const u32x4 b = pack_operand<DT>(sc[u >> 1], u & 1);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(&sVt[(32 * cb + li) * SVS + 16 * u + 8 * hh]);
        acc[cb] = Mfma<DT>::mma(a, b, acc[cb]);
      }
    }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (qi < s.lq) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* ob = reinterpret_cast<uint16_t*>(p.out) + (int64_t)(s.oq + qi) * qrs + (int64_t)h * p.d;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int c0 = 32 * cb + 8 * q4 + 4 * hh;
        if (c0 < p.d) {
          u32x2 val = {Mfma<DT>::pack2(acc[cb][4 * q4 + 0] * inv, acc[cb][4 * q4 + 1] * inv),
                       Mfma<DT>::pack2(acc[cb][4 * q4 + 2] * inv, acc[cb][4 * q4 + 3] * inv)};
          *reinterpret_cast<u32x2*>(ob + c0) = val;
        }
      }
    if (hh == 0)
      p.lse_out[(int64_t)(s.oq + qi) * p.hq + h] =
          l_tot > 0.f ? (m_run + __builtin_log2f(l_tot)) * kLn2 : -__builtin_inff();
  }
}

template <int DT, int DPAD>
static void launch_fwd_d(const AttnParams& p, bool causal, int grid, hipStream_t st) {
  if (causal) hipLaunchKernelGGL((fwd_kernel<DT, DPAD, true>), dim3(grid), dim3(256), 0, st, p);
  else hipLaunchKernelGGL((fwd_kernel<DT, DPAD, false>), dim3(grid), dim3(256), 0, st, p);
}

template <int DT>
static void launch_fwd_dt(const AttnParams& p, bool causal, int grid, hipStream_t st) {
  if (p.d <= 32) launch_fwd_d<DT, 32>(p, causal, grid, st);
  else if (p.d <= 64) launch_fwd_d<DT, 64>(p, causal, grid, st);
  else if (p.d <= 128) launch_fwd_d<DT, 128>(p, causal, grid, st);
  else launch_fwd_d<DT, 256>(p, causal, grid, st);
}

hipError_t launch_fwd(const AttnParams& p, int dtype, bool causal, int max_q_tiles, hipStream_t st) {
  const int grid = max_q_tiles * p.hq;
  if (grid <= 0) return hipSuccess;
  if (dtype == kBF16) launch_fwd_dt<kBF16>(p, causal, grid, st);
  else launch_fwd_dt<kFP16>(p, causal, grid, st);
  return hipGetLastError();
}

}  // namespace attn
