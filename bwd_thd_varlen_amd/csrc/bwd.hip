// Backward kernels.  With P recomputed from the saved LSE,
//   P = exp(scale*S - LSE),  dP = dO V^T,  dS = P o (dP - Delta),
//   dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO,
// where Delta = rowsum(dO o O) comes from the preprocess kernel.
//
// dK/dV: one workgroup per (sequence, 32*NW-key tile, KV head g).  Each wave
// owns 32 keys; K and V of those keys stay in registers (or LDS for d=256)
// for the whole workgroup, which loops over the hq/hkv query heads of g and
// over the 64-query tiles that reach the keys, in a fixed order, so the sum
// over the GQA group happens in registers: deterministic and without
// atomics (TransformerEngine issue 2448, "Expected behavior"; the KV rows of
// a tile no query reaches come out as exact zeros).
//
// dQ: one workgroup per (sequence, 128-query tile, query head): Q, dO,
// LSE and Delta of its queries stay in registers while K/V steps stream
// through LDS; S and dP are recomputed here instead of accumulating dQ across
// key-tile workgroups, which keeps every dQ element owned by one workgroup.
//
// Layout tricks are those of the forward kernel (common.h): score tiles are
// computed so that the lane index runs over the dimension that survives the
// next product, and the matching operand is read from a transposed LDS copy
// stored in perm16 order.
#include "common.h"

namespace attn {

// ----------------------------------------------------------------- dQ
template <int DT, int DPAD, bool CAUSAL>
__global__ __launch_bounds__(256, DPAD <= 128 ? 2 : 1) void dq_kernel(AttnParams p) {
  constexpr int NT = DPAD / 16;
  constexpr int NCB = DPAD / 32;
  constexpr int KS = kKVStep;
  constexpr int SRS = DPAD + 8;        // row-major K / V stride
  constexpr int STS = KS + 8;          // K^T stride
  constexpr int CPR = DPAD / 8;
  constexpr int UNITS = (KS / 4) * CPR;
  constexpr int UPT = (UNITS + 255) / 256;

  __shared__ __attribute__((aligned(16))) uint16_t sK[KS * SRS];
  __shared__ __attribute__((aligned(16))) uint16_t sV[KS * SRS];
  __shared__ __attribute__((aligned(16))) uint16_t sKt[DPAD * STS];

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
  const int64_t qoff = (int64_t)s.oq * qrs + (int64_t)h * p.d;
  const uint16_t* qb = reinterpret_cast<const uint16_t*>(p.q) + qoff;
  const uint16_t* dob = reinterpret_cast<const uint16_t*>(p.dout) + qoff;
  const uint16_t* kb = reinterpret_cast<const uint16_t*>(p.k) + (int64_t)s.ok * kvrs + (int64_t)g * p.d;
  const uint16_t* vb = reinterpret_cast<const uint16_t*>(p.v) + (int64_t)s.ok * kvrs + (int64_t)g * p.d;
  const u32x4 z4 = {0u, 0u, 0u, 0u};
  const bool qvalid = qi < s.lq;

  u32x4 qreg[NT], doreg[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int c = 16 * t + 8 * hh;
    const bool ok = qvalid && c < p.d;
    qreg[t] = ok ? ldg16(qb + (int64_t)qi * qrs + c) : z4;
    doreg[t] = ok ? ldg16(dob + (int64_t)qi * qrs + c) : z4;
  }
  const int64_t srow = (int64_t)(s.oq + qi) * p.hq + h;
  const float lse2 = qvalid ? p.lse[srow] * kLog2e : __builtin_inff();
  const float dlt = qvalid ? p.delta[srow] : 0.f;

  const int q_end = min(s.lq, m0 + kQTile);
  const int kend = CAUSAL ? min(s.lk, q_end) : s.lk;
  const int nsteps = (kend + KS - 1) / KS;
  const float sl2e = p.scale_log2e;

  f32x16 acc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) acc[cb] = zero16();

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
      for (int r = 0; r < 4; ++r) {
        *reinterpret_cast<u32x4*>(&sK[(4 * rg + r) * SRS + 8 * cc]) = pk[u][r];
        *reinterpret_cast<u32x4*>(&sV[(4 * rg + r) * SRS + 8 * cc]) = pv[u][r];
      }
      const int pos = perm16(4 * rg);
#pragma unroll
      for (int e8 = 0; e8 < 8; ++e8) {
        const int w = e8 >> 1, sh = (e8 & 1) * 16;
        const uint32_t x0 = (pk[u][0][w] >> sh) & 0xffffu, x1 = (pk[u][1][w] >> sh) & 0xffffu;
        const uint32_t x2 = (pk[u][2][w] >> sh) & 0xffffu, x3 = (pk[u][3][w] >> sh) & 0xffffu;
        u32x2 val = {x0 | (x1 << 16), x2 | (x3 << 16)};
        *reinterpret_cast<u32x2*>(&sKt[(8 * cc + e8) * STS + pos]) = val;
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
    if (wq_lo >= s.lq) continue;
    if (CAUSAL && n0 > wq_hi) continue;

    f32x16 sc[2], dp[2];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      sc[kb2] = zero16();
      dp[kb2] = zero16();
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int o = (32 * kb2 + li) * SRS + 16 * t + 8 * hh;
        sc[kb2] = Mfma<DT>::mma(*reinterpret_cast<const u32x4*>(&sK[o]), qreg[t], sc[kb2]);
        dp[kb2] = Mfma<DT>::mma(*reinterpret_cast<const u32x4*>(&sV[o]), doreg[t], dp[kb2]);
      }
    }
    const bool need_mask = CAUSAL && (n0 + KS - 1 > wq_lo);
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float pr = fast_exp2(__builtin_fmaf(sc[kb2][r], sl2e, -lse2));
        if (need_mask) {
          const int j = n0 + 32 * kb2 + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (j > qi) pr = 0.f;
        }
        sc[kb2][r] = pr * (dp[kb2][r] - dlt);     // dS
      }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const u32x4 b = pack_operand<DT>(sc[u >> 1], u & 1);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(&sKt[(32 * cb + li) * STS + 16 * u + 8 * hh]);
        acc[cb] = Mfma<DT>::mma(a, b, acc[cb]);
      }
    }
  }

  if (qvalid) {
    uint16_t* out = reinterpret_cast<uint16_t*>(p.dq) + (int64_t)(s.oq + qi) * qrs + (int64_t)h * p.d;
    const float sc0 = p.scale;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int c0 = 32 * cb + 8 * q4 + 4 * hh;
        if (c0 < p.d) {
          u32x2 val = {Mfma<DT>::pack2(acc[cb][4 * q4 + 0] * sc0, acc[cb][4 * q4 + 1] * sc0),
                       Mfma<DT>::pack2(acc[cb][4 * q4 + 2] * sc0, acc[cb][4 * q4 + 3] * sc0)};
          *reinterpret_cast<u32x2*>(out + c0) = val;
        }
      }
  }
}

// ----------------------------------------------------------------- dK / dV
// NW waves (32 keys each), BM queries per step, K/V operands in registers
// (KV_LDS = false) or re-read from LDS (KV_LDS = true, for d = 256).
template <int DT, int DPAD, bool CAUSAL, int NW, int BM, bool KV_LDS>
__global__ __launch_bounds__(NW * 64, 1) void dkdv_kernel(AttnParams p) {
  constexpr int NTH = NW * 64;
  constexpr int BN = 32 * NW;
  constexpr int NIB = BM / 32;         // 32-query blocks per step
  constexpr int NU = BM / 16;          // 16-query chunks per step
  constexpr int NT = DPAD / 16;
  constexpr int NCB = DPAD / 32;
  constexpr int SRS = DPAD + 8;        // row-major stride
  constexpr int STS = BM + 8;          // transposed stride
  constexpr int CPR = DPAD / 8;
  constexpr int UNITS = (BM / 4) * CPR;
  constexpr int UPT = (UNITS + NTH - 1) / NTH;
  constexpr int KVROWS = KV_LDS ? BN : 1;

  __shared__ __attribute__((aligned(16))) uint16_t sQ[BM * SRS];
  __shared__ __attribute__((aligned(16))) uint16_t sdO[BM * SRS];
  __shared__ __attribute__((aligned(16))) uint16_t sQt[DPAD * STS];
  __shared__ __attribute__((aligned(16))) uint16_t sdOt[DPAD * STS];
  __shared__ __attribute__((aligned(16))) float sL[BM];
  __shared__ __attribute__((aligned(16))) float sD[BM];
  __shared__ __attribute__((aligned(16))) uint16_t sK[KVROWS * SRS];
  __shared__ __attribute__((aligned(16))) uint16_t sV[KVROWS * SRS];

  const int ntiles = p.hdr[kHdrNKVTiles];
  int item, g;
  xcd_split(blockIdx.x, p.hkv, item, g);
  if (item >= ntiles) return;
  const int2 e = p.list[item];
  const SeqInfo s = p.seq[e.x];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 31, hh = lane >> 5;
  const int n0 = e.y * BN;
  const int kj = n0 + wave * 32 + li;          // this lane's key (B-operand column)
  const int wk_lo = n0 + wave * 32, wk_hi = wk_lo + 31;
  const int64_t qrs = (int64_t)p.hq * p.d, kvrs = (int64_t)p.hkv * p.d;
  const int64_t kvoff = (int64_t)s.ok * kvrs + (int64_t)g * p.d;
  const uint16_t* kb = reinterpret_cast<const uint16_t*>(p.k) + kvoff;
  const uint16_t* vb = reinterpret_cast<const uint16_t*>(p.v) + kvoff;
  const u32x4 z4 = {0u, 0u, 0u, 0u};
  const float sl2e = p.scale_log2e;

  // K and V operands of this wave's 32 keys (zero beyond the real keys)
  u32x4 kreg[KV_LDS ? 1 : NT], vreg[KV_LDS ? 1 : NT];
  if (!KV_LDS) {
#pragma unroll
    for (int t = 0; t < (KV_LDS ? 1 : NT); ++t) {
      const int c = 16 * t + 8 * hh;
      const bool ok = kj < s.lk && c < p.d;
      kreg[t] = ok ? ldg16(kb + (int64_t)kj * kvrs + c) : z4;
      vreg[t] = ok ? ldg16(vb + (int64_t)kj * kvrs + c) : z4;
    }
  } else {
    for (int unit = tid; unit < BN * CPR; unit += NTH) {
      const int r = unit / CPR, cc = unit - r * CPR;
      const int j = n0 + r;
      const bool ok = j < s.lk && 8 * cc < p.d;
      *reinterpret_cast<u32x4*>(&sK[r * SRS + 8 * cc]) = ok ? ldg16(kb + (int64_t)j * kvrs + 8 * cc) : z4;
      *reinterpret_cast<u32x4*>(&sV[r * SRS + 8 * cc]) = ok ? ldg16(vb + (int64_t)j * kvrs + 8 * cc) : z4;
    }
  }

  f32x16 adk[NCB], adv[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    adk[cb] = zero16();
    adv[cb] = zero16();
  }

  // query tiles that reach this key tile
  const int m_first = CAUSAL ? n0 / BM : 0;
  const int m_last = (s.lq + BM - 1) / BM;
  const int nm = m_last > m_first ? m_last - m_first : 0;
  const int nsteps = nm * p.group;
  const int h0 = g * p.group;

  u32x4 pq[UPT][4], pdo[UPT][4];
  float pl = 0.f;
  auto load_step = [&](int step) {
    const int hg = step / nm;
    const int m = m_first + (step - hg * nm);
    const int h = h0 + hg;
    const int i0 = m * BM;
    const int64_t base = (int64_t)s.oq * qrs + (int64_t)h * p.d;
    const uint16_t* qb = reinterpret_cast<const uint16_t*>(p.q) + base;
    const uint16_t* dob = reinterpret_cast<const uint16_t*>(p.dout) + base;
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int unit = tid + NTH * u;
      const int rg = unit / CPR, cc = unit - rg * CPR;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = i0 + 4 * rg + r;
        const bool ok = unit < UNITS && i < s.lq && 8 * cc < p.d;
        const int64_t off = (int64_t)i * qrs + 8 * cc;
        pq[u][r] = ok ? ldg16(qb + off) : z4;
        pdo[u][r] = ok ? ldg16(dob + off) : z4;
      }
    }
    // threads [0, BM) fetch LSE*log2(e), threads [BM, 2BM) fetch Delta
    if (tid < 2 * BM) {
      const int i = i0 + (tid % BM);
      const int64_t srow = (int64_t)(s.oq + i) * p.hq + h;
      if (tid < BM) pl = i < s.lq ? p.lse[srow] * kLog2e : __builtin_inff();
      else pl = i < s.lq ? p.delta[srow] : 0.f;
    }
  };
  auto store_step = [&]() {
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int unit = tid + NTH * u;
      if (UNITS % NTH != 0 && unit >= UNITS) continue;
      const int rg = unit / CPR, cc = unit - rg * CPR;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        *reinterpret_cast<u32x4*>(&sQ[(4 * rg + r) * SRS + 8 * cc]) = pq[u][r];
        *reinterpret_cast<u32x4*>(&sdO[(4 * rg + r) * SRS + 8 * cc]) = pdo[u][r];
      }
      const int pos = perm16(4 * rg);
#pragma unroll
      for (int e8 = 0; e8 < 8; ++e8) {
        const int w = e8 >> 1, sh = (e8 & 1) * 16;
        {
          const uint32_t x0 = (pq[u][0][w] >> sh) & 0xffffu, x1 = (pq[u][1][w] >> sh) & 0xffffu;
          const uint32_t x2 = (pq[u][2][w] >> sh) & 0xffffu, x3 = (pq[u][3][w] >> sh) & 0xffffu;
          u32x2 val = {x0 | (x1 << 16), x2 | (x3 << 16)};
          *reinterpret_cast<u32x2*>(&sQt[(8 * cc + e8) * STS + pos]) = val;
        }
        {
          const uint32_t x0 = (pdo[u][0][w] >> sh) & 0xffffu, x1 = (pdo[u][1][w] >> sh) & 0xffffu;
          const uint32_t x2 = (pdo[u][2][w] >> sh) & 0xffffu, x3 = (pdo[u][3][w] >> sh) & 0xffffu;
          u32x2 val = {x0 | (x1 << 16), x2 | (x3 << 16)};
          *reinterpret_cast<u32x2*>(&sdOt[(8 * cc + e8) * STS + pos]) = val;
        }
      }
    }
    if (tid < BM) sL[tid] = pl;
    else if (tid < 2 * BM) sD[tid - BM] = pl;
  };

  if (nsteps > 0) load_step(0);
  for (int step = 0; step < nsteps; ++step) {
    __syncthreads();
    store_step();
    __syncthreads();
    if (step + 1 < nsteps) load_step(step + 1);
    const int hg = step / nm;
    const int i0 = (m_first + (step - hg * nm)) * BM;
    if (wk_lo >= s.lk) continue;                  // no real key in this wave
    if (CAUSAL && i0 + BM - 1 < wk_lo) continue;  // every query precedes every key

    f32x16 sc[NIB], dp[NIB];
#pragma unroll
    for (int ib = 0; ib < NIB; ++ib) {
      sc[ib] = zero16();
      dp[ib] = zero16();
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int o = (32 * ib + li) * SRS + 16 * t + 8 * hh;
        u32x4 kop, vop;
        if (KV_LDS) {
          const int ko = (32 * wave + li) * SRS + 16 * t + 8 * hh;
          kop = *reinterpret_cast<const u32x4*>(&sK[ko]);
          vop = *reinterpret_cast<const u32x4*>(&sV[ko]);
        } else {
          kop = kreg[KV_LDS ? 0 : t];
          vop = vreg[KV_LDS ? 0 : t];
        }
        sc[ib] = Mfma<DT>::mma(*reinterpret_cast<const u32x4*>(&sQ[o]), kop, sc[ib]);
        dp[ib] = Mfma<DT>::mma(*reinterpret_cast<const u32x4*>(&sdO[o]), vop, dp[ib]);
      }
    }
    const bool need_mask = CAUSAL && (i0 < wk_hi);
#pragma unroll
    for (int ib = 0; ib < NIB; ++ib)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int ibase = 32 * ib + 8 * q4 + 4 * hh;   // first of 4 consecutive queries
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(&sL[ibase]);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(&sD[ibase]);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int r = 4 * q4 + c;
          float pr = fast_exp2(__builtin_fmaf(sc[ib][r], sl2e, -l4[c]));
          if (need_mask && kj > i0 + ibase + c) pr = 0.f;
          sc[ib][r] = pr;
          dp[ib][r] = pr * (dp[ib][r] - d4[c]);
        }
      }
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const u32x4 bp = pack_operand<DT>(sc[u >> 1], u & 1);
      const u32x4 bds = pack_operand<DT>(dp[u >> 1], u & 1);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const int o = (32 * cb + li) * STS + 16 * u + 8 * hh;
        adv[cb] = Mfma<DT>::mma(*reinterpret_cast<const u32x4*>(&sdOt[o]), bp, adv[cb]);
        adk[cb] = Mfma<DT>::mma(*reinterpret_cast<const u32x4*>(&sQt[o]), bds, adk[cb]);
      }
    }
  }

  if (kj < s.lk) {
    const int64_t row = (int64_t)kj * kvrs;
    uint16_t* dkb = reinterpret_cast<uint16_t*>(p.dk) + kvoff + row;
    uint16_t* dvb = reinterpret_cast<uint16_t*>(p.dv) + kvoff + row;
    const float sc0 = p.scale;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int c0 = 32 * cb + 8 * q4 + 4 * hh;
        if (c0 < p.d) {
          u32x2 vk = {Mfma<DT>::pack2(adk[cb][4 * q4 + 0] * sc0, adk[cb][4 * q4 + 1] * sc0),
                      Mfma<DT>::pack2(adk[cb][4 * q4 + 2] * sc0, adk[cb][4 * q4 + 3] * sc0)};
          u32x2 vv = {Mfma<DT>::pack2(adv[cb][4 * q4 + 0], adv[cb][4 * q4 + 1]),
                      Mfma<DT>::pack2(adv[cb][4 * q4 + 2], adv[cb][4 * q4 + 3])};
          *reinterpret_cast<u32x2*>(dkb + c0) = vk;
          *reinterpret_cast<u32x2*>(dvb + c0) = vv;
        }
      }
  }
}

// ----------------------------------------------------------------- launchers
template <int DT, int DPAD>
static void launch_dq_d(const AttnParams& p, bool causal, int grid, hipStream_t st) {
  if (causal) hipLaunchKernelGGL((dq_kernel<DT, DPAD, true>), dim3(grid), dim3(256), 0, st, p);
  else hipLaunchKernelGGL((dq_kernel<DT, DPAD, false>), dim3(grid), dim3(256), 0, st, p);
}

template <int DT>
static void launch_dq_dt(const AttnParams& p, bool causal, int grid, hipStream_t st) {
  if (p.d <= 32) launch_dq_d<DT, 32>(p, causal, grid, st);
  else if (p.d <= 64) launch_dq_d<DT, 64>(p, causal, grid, st);
  else if (p.d <= 128) launch_dq_d<DT, 128>(p, causal, grid, st);
  else launch_dq_d<DT, 256>(p, causal, grid, st);
}

hipError_t launch_dq(const AttnParams& p, int dtype, bool causal, int max_q_tiles, hipStream_t st) {
  const int grid = max_q_tiles * p.hq;
  if (grid <= 0) return hipSuccess;
  if (dtype == kBF16) launch_dq_dt<kBF16>(p, causal, grid, st);
  else launch_dq_dt<kFP16>(p, causal, grid, st);
  return hipGetLastError();
}

// keys per dK/dV work item for a head dim
int dkdv_tile(int d) { return d <= 128 ? 128 : 64; }

template <int DT, int DPAD, int NW, int BM, bool KVL>
static void launch_dkdv_d(const AttnParams& p, bool causal, int grid, hipStream_t st) {
  if (causal)
    hipLaunchKernelGGL((dkdv_kernel<DT, DPAD, true, NW, BM, KVL>), dim3(grid), dim3(NW * 64), 0, st, p);
  else
    hipLaunchKernelGGL((dkdv_kernel<DT, DPAD, false, NW, BM, KVL>), dim3(grid), dim3(NW * 64), 0, st, p);
}

template <int DT>
static void launch_dkdv_dt(const AttnParams& p, bool causal, int grid, hipStream_t st) {
  if (p.d <= 32) launch_dkdv_d<DT, 32, 4, 64, false>(p, causal, grid, st);
  else if (p.d <= 64) launch_dkdv_d<DT, 64, 4, 64, false>(p, causal, grid, st);
  else if (p.d <= 128) launch_dkdv_d<DT, 128, 4, 64, false>(p, causal, grid, st);
  else launch_dkdv_d<DT, 256, 2, 32, true>(p, causal, grid, st);
}

hipError_t launch_dkdv(const AttnParams& p, int dtype, bool causal, int max_kv_tiles, hipStream_t st) {
  const int grid = max_kv_tiles * p.hkv;
  if (grid <= 0) return hipSuccess;
  if (dtype == kBF16) launch_dkdv_dt<kBF16>(p, causal, grid, st);
  else launch_dkdv_dt<kFP16>(p, causal, grid, st);
  return hipGetLastError();
}

}  // namespace attn
