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
// operand of O^T = V^T P^T.  Q stays in registers for the whole tile; K and V
// arrive by global->LDS DMA into two row-major (swizzled) buffers, one step
// ahead of the compute, and V^T operands come from the LDS transpose read.
// Online softmax in the log2 domain: m = reference maximum of
// scale*log2(e)*S, l = running sum of exp2(x - m); the reference (and with it
// O and l, by exp2(m_old - m_new)) moves only when a row's maximum passes it
// by more than kRescaleSlack.
#include <type_traits>

#include "common.h"

namespace attn {

// The running maximum used as the exp2 reference only moves when a row's
// maximum exceeds it by more than this (log2 units): probabilities stay
// below 2^8 and the accumulator is rescaled rarely.  The result is the
// same softmax, since the final normalisation uses the same reference.
constexpr float kRescaleSlack = 8.0f;

// Keys per step: 32 from head dim 64 on, so that the tiles and registers of
// three workgroups fit one CU up to head dim 128 (32 KB of LDS, < 168
// VGPRs) and of two at 256 (64 KB, < 256 VGPRs); 64 for head dims up to 32.
template <int DPAD>
constexpr int fwd_step_keys() { return DPAD >= 64 ? 32 : 64; }

// DROP: dropout on the probabilities (the keep mask of dropout_block).
// F8: q and k are E4M3 codes (p.q8, p.k8): Q stays in registers as codes, K
// tiles hold DPAD code bytes per row, and S^T = K Q^T is taken on the 8-bit
// 32 x 32 x 64 product, whose result tile has the layout of the 16-bit one.
// DE: the extent of the products, at most DPAD (tiles and layouts keep the
// padded width); the k chunks and the column blocks of O past it hold no
// real column.
template <int DT, int DPAD, bool CAUSAL, bool DROP, bool F8 = false, int DE = DPAD>
__global__ __launch_bounds__(256, DPAD <= 128 ? 3 : 2) void fwd_kernel(AttnParams p) {
  // E4M3 K rows of DPAD bytes hold whole 64-code chunks of the 8-bit product
  static_assert(!F8 || DPAD >= 64, "the 8-bit scores are built for head dims 48..256");
  static_assert(DE <= DPAD, "the products cover at most the padded head dim");
  constexpr int NT = F8 ? 1 : (DE + 15) / 16;   // 16-wide k chunks of the products (16-bit Q)
  constexpr int NT8 = (DE + 63) / 64;           // 64-wide k chunks (E4M3 Q)
  constexpr int NCB = (DE + 31) / 32;           // 32-row blocks of O^T
  // keys per step (the 8-bit K tiles are half the size: 64 keys still fit
  // three workgroups per CU at head dims up to 128; 32 above, for two)
  constexpr int KS = F8 ? (DPAD <= 128 ? 64 : 32) : fwd_step_keys<DPAD>();
  constexpr int NKB = KS / 32;         // 32-key blocks of S^T per step
  // K: row reads (E4M3: DPAD bytes per row, addressed in 16-bit units)
  using LK = std::conditional_t<F8, Swz<DPAD / 2>, Swz<DPAD>>;
  using LV = Swz<DPAD>;          // V: transposed reads
  using DmaK = TileDma<LK, KS, 4>;
  using DmaV = TileDma<LV, KS, 4>;

  // two buffers of K and V (distinct arrays: their addresses are constants)
  __shared__ __attribute__((aligned(16))) uint16_t sK0[LK::template elems<KS>()];
  __shared__ __attribute__((aligned(16))) uint16_t sK1[LK::template elems<KS>()];
  __shared__ __attribute__((aligned(16))) uint16_t sV0[LV::template elems<KS>()];
  __shared__ __attribute__((aligned(16))) uint16_t sV1[LV::template elems<KS>()];
  static_assert(!DmaK::SINK && !DmaV::SINK, "these tiles split evenly over the waves");

  const int ntiles = uniform(p.hdr[kHdrNQTiles]);
  int item, h;
  xcd_split(blockIdx.x, p.hq, item, h);
  if (item >= ntiles) return;
  const WorkItem w = load_item(p.list, p.seq, item);
  const SeqInfo s = w.s;
  const int g = h / p.group;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, hh = lane >> 5;
  const int m0 = w.tile * kQTile;
  const int qi = m0 + wave * 32 + li;
  const int wq_lo = m0 + wave * 32, wq_hi = wq_lo + 31;
  // elements per row, and between consecutive tokens of a sequence
  const int64_t qrs = (int64_t)p.hq * p.d, kvrs = (int64_t)p.hkv * p.d;
  const int64_t qts = qrs * p.tsq, kvts = kvrs * p.tskv;
  const uint32_t kv_rs_bytes = (uint32_t)(kvts * 2);
  const uint32_t k_rs_bytes = F8 ? (uint32_t)kvts : kv_rs_bytes;
  const uint16_t* qb = reinterpret_cast<const uint16_t*>(p.q) + (int64_t)s.oq * qrs + (int64_t)h * p.d;
  const uint16_t* kb = reinterpret_cast<const uint16_t*>(p.k) + (int64_t)s.ok * kvrs + (int64_t)g * p.d;
  const uint8_t* qb8 = static_cast<const uint8_t*>(p.q8) + (int64_t)s.oq * qrs + (int64_t)h * p.d;
  const uint8_t* kb8 = static_cast<const uint8_t*>(p.k8) + (int64_t)s.ok * kvrs + (int64_t)g * p.d;
  const uint16_t* vb = reinterpret_cast<const uint16_t*>(p.v) + (int64_t)s.ok * kvrs + (int64_t)g * p.d;
  const u32x4 z4 = {0u, 0u, 0u, 0u};

  // key j is visible to query i iff j <= i + diag (causal)
  const int diag = CAUSAL ? s.diag : 0;
  const int q_end = min(s.lq, m0 + kQTile);
  const int kend = CAUSAL ? max(0, min(s.lk, q_end + diag)) : s.lk;
  const int nsteps = (kend + KS - 1) / KS;
  const float sl2e = p.scale_log2e;
  // the wave's queries and this lane's query shifted onto the key axis
  const int wq_lo_k = wq_lo + diag, wq_hi_k = wq_hi + diag, qi_k = qi + diag;

  DmaK dma_k;
  DmaV dma_v;
  dma_k.init(wave, lane, F8 ? p.d / 2 : p.d, k_rs_bytes);
  dma_v.init(wave, lane, p.d, kv_rs_bytes);
  auto issue = [&](int step, uint16_t* tK, uint16_t* tV) {
    const int n0 = step * KS;
    const uint16_t* krow = F8 ? reinterpret_cast<const uint16_t*>(kb8 + (int64_t)n0 * kvts)
                              : kb + (int64_t)n0 * kvts;
    dma_k.issue(krow, kend - n0, k_rs_bytes, lds_addr(tK), 0u, wave);
    dma_v.issue(vb + (int64_t)n0 * kvts, kend - n0, kv_rs_bytes, lds_addr(tV), 0u, wave);
  };
  if (nsteps > 0) issue(0, sK0, sV0);

  u32x4 qreg[NT];
  u32x4 q8lo[F8 ? NT8 : 1], q8hi[F8 ? NT8 : 1];   // E4M3 Q: codes 64 t + 32 hh + (0..31)
  if constexpr (F8) {
#pragma unroll
    for (int t = 0; t < NT8; ++t) {
      const int c = 64 * t + 32 * hh;
      q8lo[t] = (qi < s.lq && c < p.d) ? ldg16(qb8 + (int64_t)qi * qts + c) : z4;
      q8hi[t] = (qi < s.lq && c + 16 < p.d) ? ldg16(qb8 + (int64_t)qi * qts + c + 16) : z4;
    }
  } else {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int c = 16 * t + 8 * hh;
      qreg[t] = (qi < s.lq && c < p.d) ? ldg16(qb + (int64_t)qi * qts + c) : z4;
    }
  }
  wait_vm<0>();   // Q and the first step's tiles; keeps the compiler from re-waiting in the loop

  f32x16 acc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) acc[cb] = zero16();
  float m_run = -__builtin_inff(), l_run = 0.f;

  SwzRowReader<DPAD> rk(lane);   // K rows (16-bit K)
  SwzTrReader<DPAD> rtv(lane);   // V, transposed
  // One barrier per step: after it, every wave has finished step - 1, so the
  // DMA of step + 1 can refill that step's buffer.
  auto do_step = [&](int step, const uint16_t* tK, const uint16_t* tV, uint16_t* nK, uint16_t* nV) {
    rk.refresh();
    rtv.refresh();
    wait_vm<0>();                                // this step's tiles have landed
    barrier_lds_dma();
    if (step + 1 < nsteps) issue(step + 1, nK, nV);
    const int n0 = step * KS;
    // waves with no real query, or whose queries all precede the step, idle
    if (wq_lo < s.lq && !(CAUSAL && n0 > wq_hi_k)) {
      f32x16 sc[NKB];
#pragma unroll
      for (int kb2 = 0; kb2 < NKB; ++kb2) {
        sc[kb2] = zero16();
        if constexpr (F8) {
          // key row 32 kb2 + li, code bytes 64 t + 32 hh .. +32 (16-bit columns 32 t + 16 hh)
#pragma unroll
          for (int t = 0; t < NT8; ++t) {
            sc[kb2] = mma_e4m3(lds_row8<LK>(tK, 32 * kb2 + li, 32 * t + 16 * hh),
                               lds_row8<LK>(tK, 32 * kb2 + li, 32 * t + 16 * hh + 8),
                               q8lo[t], q8hi[t], sc[kb2]);
          }
        } else {
          // K operands read two MFMAs ahead, pinned with scheduling barriers
          constexpr int PD = 2;
          u32x4 ak[NT];
#pragma unroll
          for (int t = 0; t < PD; ++t) ak[t] = rk.read(lds_addr(tK), kb2, t);
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            __builtin_amdgcn_sched_barrier(0);
            sc[kb2] = Mfma<DT>::mma(ak[t], qreg[t], sc[kb2]);
            if (t + PD < NT) ak[t + PD] = rk.read(lds_addr(tK), kb2, t + PD);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      const bool need_mask = (n0 + KS > kend) || (CAUSAL && n0 + KS - 1 > wq_lo_k);
      if (need_mask) {
#pragma unroll
        for (int kb2 = 0; kb2 < NKB; ++kb2)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = n0 + 32 * kb2 + 8 * (r >> 2) + 4 * hh + (r & 3);
            if (j >= kend || (CAUSAL && j > qi_k)) sc[kb2][r] = -__builtin_inff();
          }
      }
      const float mx = max_halves(tree_max(sc)) * sl2e;
      // the exp2 reference moves only when a row's maximum exceeds it by
      // more than kRescaleSlack, so O is rarely rescaled
      const bool move = mx > m_run + kRescaleSlack;
      if (__any(move)) {
        const float m_new = move ? mx : m_run;
        // 1 for lanes that keep their reference (also when it is still -inf),
        // 0 for a lane whose first finite maximum arrives
        const float alpha = move ? fast_exp2(m_run - m_new) : 1.f;
        l_run *= alpha;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[cb][r] *= alpha;
        m_run = m_new;
      }
      const float base = (m_run == -__builtin_inff()) ? 0.f : m_run;
#pragma unroll
      for (int kb2 = 0; kb2 < NKB; ++kb2)
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[kb2][r] = fast_exp2(__builtin_fmaf(sc[kb2][r], sl2e, -base));
      l_run += tree_sum(sc);   // the softmax's own sum: before dropout
      if constexpr (DROP) {
        // this lane's query row of the 4 x 4 blocks at keys 8g + 4hh (+0..3)
#pragma unroll
        for (int kb2 = 0; kb2 < NKB; ++kb2)
          dropout_row16(p, w.b, h, qi >> 2, (n0 + 32 * kb2 + 4 * hh) >> 2, li & 3, 1.f, sc[kb2]);
      }
#pragma unroll
      for (int u = 0; u < 2 * NKB; ++u) {
        const u32x4 b = pack_operand<DT>(sc[u >> 1], u & 1);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
          acc[cb] = Mfma<DT>::mma(rtv.read(lds_addr(tV), cb, u), b, acc[cb]);
      }
    }
  };
  for (int step = 0; step < nsteps; step += 2) {
    do_step(step, sK0, sV0, sK1, sV1);
    if (step + 1 < nsteps) do_step(step + 1, sK1, sV1, sK0, sV0);
  }

  const float l_tot = sum_halves(l_run);
  if (qi < s.lq) {
    const float inv = l_tot > 0.f ? (DROP ? p.drop_scale : 1.f) * p.out_scale / l_tot : 0.f;
    const int64_t row = (int64_t)s.oq + (int64_t)qi * p.tsq;
    uint16_t* ob = reinterpret_cast<uint16_t*>(p.out) + row * qrs + (int64_t)h * p.d;
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
      p.lse_out[row * p.hq + h] =
          l_tot > 0.f ? ((m_run == -__builtin_inff() ? 0.f : m_run) + __builtin_log2f(l_tot)) * kLn2
                      : -__builtin_inff();
  }
}

template <int DT, int DPAD, int DE>
static void launch_fwd_d(const AttnParams& p, bool causal, int grid, hipStream_t st) {
  if constexpr (DPAD >= 64) {
    if (p.q8) {   // E4M3 q and k (no dropout on this path)
      if (causal) hipLaunchKernelGGL((fwd_kernel<DT, DPAD, true, false, true, DE>), dim3(grid), dim3(256), 0, st, p);
      else hipLaunchKernelGGL((fwd_kernel<DT, DPAD, false, false, true, DE>), dim3(grid), dim3(256), 0, st, p);
      return;
    }
  }
  const bool drop = p.drop_t != 0;
  if (causal && drop) hipLaunchKernelGGL((fwd_kernel<DT, DPAD, true, true, false, DE>), dim3(grid), dim3(256), 0, st, p);
  else if (causal) hipLaunchKernelGGL((fwd_kernel<DT, DPAD, true, false, false, DE>), dim3(grid), dim3(256), 0, st, p);
  else if (drop) hipLaunchKernelGGL((fwd_kernel<DT, DPAD, false, true, false, DE>), dim3(grid), dim3(256), 0, st, p);
  else hipLaunchKernelGGL((fwd_kernel<DT, DPAD, false, false, false, DE>), dim3(grid), dim3(256), 0, st, p);
}

// the extent of the products: the head dim rounded up to 16
template <int DT>
static void launch_fwd_dt(const AttnParams& p, bool causal, int grid, hipStream_t st) {
  switch ((p.d + 15) >> 4) {
    case 1: case 2: launch_fwd_d<DT, 32, 32>(p, causal, grid, st); break;
    case 3: launch_fwd_d<DT, 64, 48>(p, causal, grid, st); break;
    case 4: launch_fwd_d<DT, 64, 64>(p, causal, grid, st); break;
    case 5: launch_fwd_d<DT, 128, 80>(p, causal, grid, st); break;
    case 6: launch_fwd_d<DT, 128, 96>(p, causal, grid, st); break;
    case 7: launch_fwd_d<DT, 128, 112>(p, causal, grid, st); break;
    case 8: launch_fwd_d<DT, 128, 128>(p, causal, grid, st); break;
    case 9: launch_fwd_d<DT, 256, 144>(p, causal, grid, st); break;
    case 10: launch_fwd_d<DT, 256, 160>(p, causal, grid, st); break;
    case 11: launch_fwd_d<DT, 256, 176>(p, causal, grid, st); break;
    case 12: launch_fwd_d<DT, 256, 192>(p, causal, grid, st); break;
    case 13: launch_fwd_d<DT, 256, 208>(p, causal, grid, st); break;
    case 14: launch_fwd_d<DT, 256, 224>(p, causal, grid, st); break;
    case 15: launch_fwd_d<DT, 256, 240>(p, causal, grid, st); break;
    default: launch_fwd_d<DT, 256, 256>(p, causal, grid, st);
  }
}

hipError_t launch_fwd(const AttnParams& p, int dtype, bool causal, int max_q_tiles, hipStream_t st) {
  const int grid = max_q_tiles * p.hq;
  if (grid <= 0) return hipSuccess;
  if (dtype == kBF16) launch_fwd_dt<kBF16>(p, causal, grid, st);
  else launch_fwd_dt<kFP16>(p, causal, grid, st);
  return hipGetLastError();
}

}  // namespace attn
