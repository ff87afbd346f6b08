// Backward kernels.  With P recomputed from the saved LSE,
//   P = exp(scale*S - LSE),  dP = dO V^T,  dS = P o (dP - Delta),
//   dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO,
// where Delta = rowsum(dO o O) is formed in the dQ kernel's prologue, which
// also stores -Delta and LSE*log2(e) per (row, head) for dK/dV.
//
// dK/dV: one workgroup per (sequence, 128-key tile, KV head g).  Each wave
// owns 32 keys (head dims above 128: two waves own 32 keys, one half of the
// head dim each); K and V of those keys stay in registers for the whole
// workgroup, which loops over the hq/hkv query heads of g and over the query
// tiles that reach the keys, in a fixed order, so the sum over the GQA group
// happens in registers: deterministic and without atomics (TransformerEngine
// issue 2448, "Expected behavior"; the KV rows of a tile no query reaches
// come out as exact zeros).
//
// dQ: one workgroup per (sequence, 128-query tile, query head): Q, dO,
// LSE and Delta of its queries stay in registers while K/V steps stream
// through LDS (head dims above 192: two waves per 32 queries, one holding Q
// and one dO, each accumulating half of dQ); S and dP are recomputed here
// instead of accumulating dQ across key-tile workgroups, which keeps every dQ
// element owned by one workgroup.
//
// Both kernels fill LDS tiles by global->LDS DMA ahead of the compute (see
// TileDma in common.h): dQ double-buffers one step ahead, dK/dV uses a ring
// (the split kernels, one workgroup per CU, a ring of three with half their
// waves half a step behind the others).
//
// Layout tricks are those of the forward kernel (common.h): score tiles are
// computed so that the lane index runs over the dimension that survives the
// next product, and the operand that contracts over a tile's rows is read
// from the same row-major LDS tile with the transpose read.
//
// Head dims below the padded tile width (32, 64, 128, 192 or 256 columns):
// the products run over the head dim rounded up to 16 and skip the column
// blocks of the outputs past it, whose operands are zero (the split kernels
// keep their output blocks in pairs).
#include "common.h"

namespace attn {

// x[0..3] += the four values stored at w (accumulating backward): the sum is
// formed in fp32 and rounded once.
template <int DT>
__device__ __forceinline__ void add_stored(float* x, u32x2 w) {
  const f32x2 a = Mfma<DT>::unpack2(w[0]), b = Mfma<DT>::unpack2(w[1]);
  x[0] += a[0];
  x[1] += a[1];
  x[2] += b[0];
  x[3] += b[1];
}

// One row (of dQ, dK or dV) over column blocks [cb0, cb0 + nb) of the head
// dim (nb <= NB), times `mul` and rounded once (ACC: added to what `out`
// holds); `out` is the row of the head, lane half hh holds columns 4 hh .. +3
// of each 8-column group.
template <int DT, bool ACC, int NB>
__device__ __forceinline__ void store_row(const AttnParams& p, uint16_t* out, int cb0, int hh,
                                          const f32x16 (&acc)[NB], float mul, int nb = NB) {
#pragma unroll
  for (int cb = 0; cb < NB; ++cb)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int c0 = 32 * (cb0 + cb) + 8 * q4 + 4 * hh;
      if (cb < nb && c0 < p.d) {
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = acc[cb][4 * q4 + e] * mul;
        if constexpr (ACC) add_stored<DT>(x, *reinterpret_cast<const u32x2*>(out + c0));
        u32x2 val = {Mfma<DT>::pack2(x[0], x[1]), Mfma<DT>::pack2(x[2], x[3])};
        *reinterpret_cast<u32x2*>(out + c0) = val;
      }
    }
}

// dQ of this lane's query: the row scaled by the softmax scale
template <int DT, bool ACC, int NB>
__device__ __forceinline__ void store_dq(const AttnParams& p, uint16_t* out, int cb0, int hh,
                                         const f32x16 (&acc)[NB], int nb = NB) {
  store_row<DT, ACC, NB>(p, out, cb0, hh, acc, p.scale, nb);
}

// One fp32 row (unscaled) into a partial plane of a split GQA group.
template <int NB>
__device__ __forceinline__ void store_row_part(const AttnParams& p, float* out, int hh, const f32x16 (&acc)[NB]) {
#pragma unroll
  for (int cb = 0; cb < NB; ++cb)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int c0 = 32 * cb + 8 * q4 + 4 * hh;
      if (c0 < p.d)
        *reinterpret_cast<f32x4*>(out + c0) =
            (f32x4){acc[cb][4 * q4], acc[cb][4 * q4 + 1], acc[cb][4 * q4 + 2], acc[cb][4 * q4 + 3]};
    }
}

// dK (scaled) and dV of this lane's key over column blocks [cb0, cb0 + nb)
// (nb <= NB), rounded once (ACC: added to what the rows hold); dkb / dvb are the key's
// rows of the KV head.
template <int DT, bool ACC, int NB>
__device__ __forceinline__ void store_dkdv(const AttnParams& p, uint16_t* dkb, uint16_t* dvb, int cb0, int hh,
                                           const f32x16 (&adk)[NB], const f32x16 (&adv)[NB], int nb = NB) {
  const float sc0 = p.scale;
#pragma unroll
  for (int cb = 0; cb < NB; ++cb)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int c0 = 32 * (cb0 + cb) + 8 * q4 + 4 * hh;
      if (cb < nb && c0 < p.d) {
        float xk[4], xv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xk[e] = adk[cb][4 * q4 + e] * sc0;
          xv[e] = adv[cb][4 * q4 + e];
        }
        if constexpr (ACC) {
          add_stored<DT>(xk, *reinterpret_cast<const u32x2*>(dkb + c0));
          add_stored<DT>(xv, *reinterpret_cast<const u32x2*>(dvb + c0));
        }
        u32x2 vk = {Mfma<DT>::pack2(xk[0], xk[1]), Mfma<DT>::pack2(xk[2], xk[3])};
        u32x2 vv = {Mfma<DT>::pack2(xv[0], xv[1]), Mfma<DT>::pack2(xv[2], xv[3])};
        *reinterpret_cast<u32x2*>(dkb + c0) = vk;
        *reinterpret_cast<u32x2*>(dvb + c0) = vv;
      }
    }
}

// This workgroup's fp32 dK and dV of this lane's key (unscaled) over column
// blocks [cb0, cb0 + nb) (nb <= NB), into its partial planes (split GQA group).
template <int NB>
__device__ __forceinline__ void store_dkdv_part(const AttnParams& p, float* dkp, float* dvp, int cb0, int hh,
                                                const f32x16 (&adk)[NB], const f32x16 (&adv)[NB],
                                                int nb = NB) {
#pragma unroll
  for (int cb = 0; cb < NB; ++cb)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int c0 = 32 * (cb0 + cb) + 8 * q4 + 4 * hh;
      if (cb < nb && c0 < p.d) {
        *reinterpret_cast<f32x4*>(dkp + c0) =
            (f32x4){adk[cb][4 * q4], adk[cb][4 * q4 + 1], adk[cb][4 * q4 + 2], adk[cb][4 * q4 + 3]};
        *reinterpret_cast<f32x4*>(dvp + c0) =
            (f32x4){adv[cb][4 * q4], adv[cb][4 * q4 + 1], adv[cb][4 * q4 + 2], adv[cb][4 * q4 + 3]};
      }
    }
}

// ----------------------------------------------------------------- dQ
// ACC: add into dq (the chunked, accumulating backward) instead of writing it;
// DROP: dropout on the probabilities (the keep mask of dropout_block); DE:
// the head dim rounded up to 16, the extent of the products (tiles and
// layouts keep the padded width DPAD)
template <int DT, int DPAD, bool CAUSAL, bool ACC, bool DROP, int DE>
__global__ __launch_bounds__(256, 2) void dq_kernel(AttnParams p) {
  static_assert(DE <= DPAD, "the products cover at most the padded head dim");
  constexpr int NT = (DE + 15) / 16;   // 16-wide k chunks of the products
  constexpr int NCB = (DE + 31) / 32;  // 32-column blocks of dQ
  // keys per step: 64 up to d = 128; 32 at the 192-wide tiles, so that two
  // workgroups still fit a CU's LDS
  constexpr int KS = DPAD <= 128 ? kKVStep : 32;
  constexpr int NKB = KS / 32;         // 32-key halves per step
  using LK = Lay<DPAD, true>;          // K: row reads (S) and transposed reads (dQ)
  // V: row reads (dP); at the 192-wide tiles in K's layout, so that both
  // tiles' DMA share one set of lane offsets (registers are that tight there)
  using LV = std::conditional_t<DPAD == 192, Lay<DPAD, true>, Lay<DPAD, false>>;
  using DmaK = TileDma<LK, KS, 4>;
  using DmaV = TileDma<LV, KS, 4>;

  __shared__ __attribute__((aligned(16))) uint16_t sK[2][LK::template elems<KS>()];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][LV::template elems<KS>()];

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
  const int64_t qoff = (int64_t)s.oq * qrs + (int64_t)h * p.d;
  const uint16_t* qb = reinterpret_cast<const uint16_t*>(p.q) + qoff;
  const uint16_t* dob = reinterpret_cast<const uint16_t*>(p.dout) + qoff;
  const uint16_t* kb = reinterpret_cast<const uint16_t*>(p.k) + (int64_t)s.ok * kvrs + (int64_t)g * p.d;
  const uint16_t* vb = reinterpret_cast<const uint16_t*>(p.v) + (int64_t)s.ok * kvrs + (int64_t)g * p.d;
  const u32x4 z4 = {0u, 0u, 0u, 0u};
  const bool qvalid = qi < s.lq;

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
  dma_k.init(wave, lane, p.d, kv_rs_bytes);
  dma_v.init(wave, lane, p.d, kv_rs_bytes);
  auto issue = [&](int step) {
    const uint32_t buf = (uint32_t)(step & 1);
    const int n0 = step * KS;
    // each step waits for all of the wave's DMAs, so the waves need not
    // issue equal counts: no sink DMAs
    dma_k.issue_exact(kb + (int64_t)n0 * kvts, kend - n0, kv_rs_bytes, lds_addr(sK[0]) + buf * sizeof(sK[0]), wave);
    dma_v.issue_exact(vb + (int64_t)n0 * kvts, kend - n0, kv_rs_bytes, lds_addr(sV[0]) + buf * sizeof(sV[0]), wave);
  };
  if (nsteps > 0) issue(0);

  // Q and dO of this lane's query (half hh of the head dim) stay in
  // registers; O is read once for the backward's preprocess:
  // Delta = sum_c dO_c O_c, in fp32, over the two halves of the wave
  const uint16_t* obase = reinterpret_cast<const uint16_t*>(p.o) + qoff;
  u32x4 qreg[NT], doreg[NT];
  float dpart = 0.f;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int c = 16 * t + 8 * hh;
    const bool ok = qvalid && c < p.d;
    qreg[t] = ok ? ldg16(qb + (int64_t)qi * qts + c) : z4;
    doreg[t] = ok ? ldg16(dob + (int64_t)qi * qts + c) : z4;
    const u32x4 o4 = ok ? ldg16(obase + (int64_t)qi * qts + c) : z4;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t dw = doreg[t][e], ow = o4[e];
      const f32x2 x = Mfma<DT>::unpack2(dw), y = Mfma<DT>::unpack2(ow);
      dpart = __builtin_fmaf(x[0], y[0], dpart);
      dpart = __builtin_fmaf(x[1], y[1], dpart);
    }
  }
  const int64_t qrow = (int64_t)s.oq + (int64_t)qi * p.tsq;
  const int64_t srow = qrow * p.hq + h;
  const float delta = sum_halves(dpart) * p.delta_scale;
  const float lse2 = qvalid ? p.lse[srow] * kLog2e : __builtin_inff();
  const float dlt = qvalid ? delta : 0.f;
  // the dK/dV kernel (launched next) reads both per (row, head), Delta
  // negated (its dP accumulators start from it); each is written by the one
  // work item that owns the row
  if (qvalid && hh == 0) {
    p.delta[srow] = -delta;
    p.lse2[srow] = lse2;
  }
  wait_vm<0>();

  f32x16 acc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) acc[cb] = zero16();

  // one barrier per step, as in the forward kernel
  for (int step = 0; step < nsteps; ++step) {
    wait_vm<0>();
    barrier_lds_dma();
    if (step + 1 < nsteps) issue(step + 1);
    const uint32_t tk = lds_addr(sK[0]) + (uint32_t)(step & 1) * (uint32_t)sizeof(sK[0]);
    const uint32_t tv = lds_addr(sV[0]) + (uint32_t)(step & 1) * (uint32_t)sizeof(sV[0]);
    const RowReader<LK> rk(tk, lane);
    const RowReader<LV> rv(tv, lane);
    const TrReader<LK> trk(tk, lane);
    const int n0 = step * KS;
    if (wq_lo < s.lq && !(CAUSAL && n0 > wq_hi_k)) {
      // the causal mask only on steps that touch the diagonal (a wave-uniform
      // branch): key n0 + j is hidden from this lane's query while j > qk
      const bool diag_step = CAUSAL && n0 + KS - 1 > wq_lo_k;
      const int qk = qi_k - n0;
      // the step's 32-key halves one after the other (S, dP -> dS -> dQ
      // part), so that only one half's score tiles are live at a time
#pragma unroll
      for (int kb2 = 0; kb2 < NKB; ++kb2) {
        // dP accumulates onto -Delta (without dropout, which scales dP
        // alone), so the chain ends at dP - Delta
        f32x16 sc = zero16(), dp = zero16();
        if constexpr (!DROP) {
#pragma unroll
          for (int r = 0; r < 16; ++r) dp[r] = -dlt;
        }
        // the product phases run at raised wave priority, so a wave that
        // reaches them issues its MFMAs ahead of the other waves' softmax
        // arithmetic, which then fills the matrix pipe's shadow
        __builtin_amdgcn_s_setprio(1);
        if constexpr (DPAD >= 128 && DE <= 176) {
          // S and dP interleaved, each K / V operand read two MFMAs ahead
          // (pinned with scheduling barriers; left to itself the scheduler
          // waits on each read just before its MFMA); one ahead above 160
          // columns, where Q, dO and the dQ accumulator leave no room for more
          // (at 192 the operands are left to the scheduler, which keeps the
          // DMA lane offsets in registers)
          constexpr int PD = DE > 160 ? 1 : 2;
          u32x4 ak[NT], av[NT];
#pragma unroll
          for (int t = 0; t < PD; ++t) {
            ak[t] = rk.read(kb2, t);
            av[t] = rv.read(kb2, t);
          }
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            __builtin_amdgcn_sched_barrier(0);
            sc = Mfma<DT>::mma(ak[t], qreg[t], sc);
            if (t + PD < NT) ak[t + PD] = rk.read(kb2, t + PD);
            __builtin_amdgcn_sched_barrier(0);
            dp = Mfma<DT>::mma(av[t], doreg[t], dp);
            if (t + PD < NT) av[t + PD] = rv.read(kb2, t + PD);
          }
          __builtin_amdgcn_sched_barrier(0);
        } else {
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            sc = Mfma<DT>::mma(rk.read(kb2, t), qreg[t], sc);
            dp = Mfma<DT>::mma(rv.read(kb2, t), doreg[t], dp);
          }
          // both chains end here: in the loop without the causal branch the
          // scheduler otherwise defers the dP products behind the softmax, and
          // at 192 columns Q and dO then spill and are reloaded every step
          if constexpr (DPAD == 192) asm volatile("" : "+v"(sc), "+v"(dp));
        }
        __builtin_amdgcn_s_setprio(0);
        if constexpr (DROP) {
          // dP = D o (dO V^T): dropped elements 0, kept ones scaled
          dropout_row16(p, w.b, h, qi >> 2, (n0 + 32 * kb2 + 4 * hh) >> 2, li & 3, p.drop_scale, dp);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[r] = fast_exp2(__builtin_fmaf(sc[r], sl2e, -lse2));
        if (diag_step) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (32 * kb2 + 8 * (r >> 2) + 4 * hh + (r & 3) > qk) sc[r] = 0.f;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[r] = DROP ? sc[r] * (dp[r] - dlt) : sc[r] * dp[r];     // dS
        const u32x4 b0 = pack_operand<DT>(sc, 0), b1 = pack_operand<DT>(sc, 1);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
          acc[cb] = Mfma<DT>::mma(trk.read(cb, 2 * kb2), b0, acc[cb]);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
          acc[cb] = Mfma<DT>::mma(trk.read(cb, 2 * kb2 + 1), b1, acc[cb]);
        __builtin_amdgcn_s_setprio(0);
      }
    }
  }

  if (qvalid)
    store_dq<DT, ACC>(p, reinterpret_cast<uint16_t*>(p.dq) + qrow * qrs + (int64_t)h * p.d, 0, hh, acc);
}

// ----------------------------------------------------------------- dQ, head dims 200..256
// Q, dO and the fp32 dQ accumulator of 32 queries outgrow 256 registers at
// these head dims (up to 192 dq_kernel runs on 192-wide tiles), and 64-key
// K / V tiles at d = 256 take 141 KB of LDS: one wave per SIMD.  Here
// eight waves share the 128-query tile: waves 2 qb and 2 qb + 1 own query
// block qb and split the head dim of dQ between them (64 accumulator
// registers each).  Each 32-key step, wave 2 qb forms S^T = K Q^T from Q and
// wave 2 qb + 1 forms dP^T = V dO^T (onto -Delta) from dO, each over the whole
// head dim; both tiles go through LDS, so the pair forms the same dS and each
// adds dS K over its own four column blocks.  K and V use the same padded
// tile layout; both waves of a pair form Delta from dO and O (the same
// arithmetic, so the same value).  Two barriers per step: the ring's, and the
// one after the tiles are written; waves 4..7 run half a step behind waves
// 0..3 (below).  DE: the extent of the S / dP products
// (the head dim rounded up to 16); dQ covers it in an even count of
// 32-column blocks.
template <int DT, bool CAUSAL, bool ACC, bool DROP, int DE>
__global__ __launch_bounds__(512, 1) void dq_split_kernel(AttnParams p) {
  constexpr int DPAD = 256, NW = 8, KS = 32;
  static_assert(DE % 16 == 0 && DE > 128 && DE <= DPAD, "products over whole 16-wide k chunks");
  constexpr int NT = DE / 16;          // 16-wide k chunks of the S / dP products
  // 32-column blocks of dQ: an even count, so that the two waves of a pair
  // take equal shares (a block past the head dim adds zeros)
  constexpr int NCB = 2 * ((DE + 63) / 64);
  constexpr int NCBH = NCB / 2;        // blocks of each wave of a pair
  using LK = Lay<DPAD, true>;          // K and V: row reads (S, dP); K also transposed (dQ)
  using Dma = TileDma<LK, KS, NW>;
  constexpr int NBUF = 3;
  constexpr int DMA_PER_STEP = 2 * Dma::PER_WAVE;

  __shared__ __attribute__((aligned(16))) uint16_t sK[NBUF][LK::template elems<KS>()];
  __shared__ __attribute__((aligned(16))) uint16_t sV[NBUF][LK::template elems<KS>()];
  __shared__ __attribute__((aligned(16))) uint16_t sSink[Dma::SINK ? 512 : 8];
  // the S^T (even wave) and dP^T (odd wave) tiles of each query block, as the
  // 16 accumulator registers of every lane: [wave][register / 4][lane]
  __shared__ __attribute__((aligned(16))) f32x4 sX[NW][4][64];

  const int ntiles = uniform(p.hdr[kHdrNQTiles]);
  int item, h;
  xcd_split(blockIdx.x, p.hq, item, h);
  if (item >= ntiles) return;
  const WorkItem w = load_item(p.list, p.seq, item);
  const SeqInfo s = w.s;
  const int g = h / p.group;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qblk = wave >> 1, half = wave & 1;
  const int li = lane & 31, hh = lane >> 5;
  const int m0 = w.tile * kQTile;
  const int qi = m0 + qblk * 32 + li;
  const int wq_lo = m0 + qblk * 32, wq_hi = wq_lo + 31;
  const int64_t qrs = (int64_t)p.hq * p.d, kvrs = (int64_t)p.hkv * p.d;
  const int64_t qts = qrs * p.tsq, kvts = kvrs * p.tskv;
  const uint32_t kv_rs_bytes = (uint32_t)(kvts * 2);
  const int64_t qoff = (int64_t)s.oq * qrs + (int64_t)h * p.d;
  const uint16_t* qb = reinterpret_cast<const uint16_t*>(p.q) + qoff;
  const uint16_t* dob = reinterpret_cast<const uint16_t*>(p.dout) + qoff;
  const uint16_t* obase = reinterpret_cast<const uint16_t*>(p.o) + qoff;
  const uint16_t* kb = reinterpret_cast<const uint16_t*>(p.k) + (int64_t)s.ok * kvrs + (int64_t)g * p.d;
  const uint16_t* vb = reinterpret_cast<const uint16_t*>(p.v) + (int64_t)s.ok * kvrs + (int64_t)g * p.d;
  const u32x4 z4 = {0u, 0u, 0u, 0u};
  const bool qvalid = qi < s.lq;

  const int diag = CAUSAL ? s.diag : 0;
  const int q_end = min(s.lq, m0 + kQTile);
  const int kend = CAUSAL ? max(0, min(s.lk, q_end + diag)) : s.lk;
  const int nsteps = (kend + KS - 1) / KS;
  const float sl2e = p.scale_log2e;
  const int wq_lo_k = wq_lo + diag, wq_hi_k = wq_hi + diag, qi_k = qi + diag;

  Dma dma;
  dma.init(wave, lane, p.d, kv_rs_bytes);
  // every wave issues the same number of DMAs per tile (sink DMAs fill up
  // the uneven split), so that each can wait for a given step's share
  auto issue = [&](int step, uint32_t buf) {
    const int n0 = step * KS;
    dma.issue(kb + (int64_t)n0 * kvts, kend - n0, kv_rs_bytes, lds_addr(sK[0]) + buf * (uint32_t)sizeof(sK[0]),
              lds_addr(sSink), wave);
    dma.issue(vb + (int64_t)n0 * kvts, kend - n0, kv_rs_bytes, lds_addr(sV[0]) + buf * (uint32_t)sizeof(sV[0]),
              lds_addr(sSink), wave);
  };
  // waves 4..7 run half a step behind waves 0..3 (see the loop)
  const int late = wave >= NW / 2 ? 1 : 0;
  for (int j = 0; j <= late; ++j)
    if (j < nsteps) issue(j, (uint32_t)j);
  // ring buffer of the next tile this wave issues
  uint32_t ibuf = (uint32_t)late + 1u;

  // this wave's operand (Q on even waves, dO on odd) stays in registers;
  // Delta = sum_c dO_c O_c in fp32 over the two halves of the wave
  u32x4 opreg[NT];
  float dpart = 0.f;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int c = 16 * t + 8 * hh;
    const bool ok = qvalid && c < p.d;
    const u32x4 d4 = ok ? ldg16(dob + (int64_t)qi * qts + c) : z4;
    const u32x4 o4 = ok ? ldg16(obase + (int64_t)qi * qts + c) : z4;
    opreg[t] = half ? d4 : (ok ? ldg16(qb + (int64_t)qi * qts + c) : z4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const f32x2 x = Mfma<DT>::unpack2(d4[e]), y = Mfma<DT>::unpack2(o4[e]);
      dpart = __builtin_fmaf(x[0], y[0], dpart);
      dpart = __builtin_fmaf(x[1], y[1], dpart);
    }
  }
  const int64_t qrow = (int64_t)s.oq + (int64_t)qi * p.tsq;
  const int64_t srow = qrow * p.hq + h;
  const float delta = sum_halves(dpart) * p.delta_scale;
  const float lse2 = qvalid ? p.lse[srow] * kLog2e : __builtin_inff();
  const float dlt = qvalid ? delta : 0.f;
  // for the dK/dV kernel (launched next): -Delta and LSE*log2(e) per (row,
  // head), written by the odd wave of the pair that owns the row
  if (qvalid && hh == 0 && half) {
    p.delta[srow] = -delta;
    p.lse2[srow] = lse2;
  }
  wait_vm<0>();

  f32x16 acc[NCBH];
#pragma unroll
  for (int cb = 0; cb < NCBH; ++cb) acc[cb] = zero16();
  // this wave's column blocks of dQ: cb0 .. cb0 + nb - 1
  const int cb0 = half * NCBH;
  const int nb = half ? NCB - NCBH : NCBH;

  // Waves 4..7 (query blocks 2, 3) run half a step behind waves 0..3, as in
  // dkdv_split_kernel: one barrier more before the loop (waves 0..3 one after
  // it), each wave issuing its share of a K / V tile at the start of its own
  // step (early waves tile step + 1, late ones step + 2) and waiting for it
  // before the barrier that precedes the tile's first read; a ring of three.
  if (late) {
    wait_vm_steps<DMA_PER_STEP, NBUF - 2>(min(NBUF - 2, nsteps - 1));
    barrier_lds_writes();
  }
  for (int step = 0; step < nsteps; ++step) {
    // early waves: this step's tile has landed; late waves: the early waves'
    // S^T / dP^T tiles are in LDS
    if (!late) wait_vm<0>();
    barrier_lds_writes();
    if (step + 1 + late < nsteps) issue(step + 1 + late, ibuf);
    ibuf = ibuf == NBUF - 1 ? 0u : ibuf + 1u;
    const int buf = step % NBUF;
    const uint32_t tk = lds_addr(sK[0]) + (uint32_t)buf * (uint32_t)sizeof(sK[0]);
    const uint32_t tv = lds_addr(sV[0]) + (uint32_t)buf * (uint32_t)sizeof(sV[0]);
    const int n0 = step * KS;
    // both waves of a query block are active or idle together
    const bool active = wq_lo < s.lq && !(CAUSAL && n0 > wq_hi_k);
    if (active) {
      // S^T (even wave) or dP^T onto -Delta (odd wave; without dropout, which
      // scales dP alone), each K / V operand read two MFMAs ahead
      constexpr int PD = 2;
      const RowReader<LK> rd(half ? tv : tk, lane);
      f32x16 t16 = zero16();
      if (half && !DROP) {
#pragma unroll
        for (int r = 0; r < 16; ++r) t16[r] = -dlt;
      }
      u32x4 a[NT];
#pragma unroll
      for (int t = 0; t < PD; ++t) a[t] = rd.read(0, t);
      // the product phases at raised wave priority, as in dq_kernel
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        __builtin_amdgcn_sched_barrier(0);
        t16 = Mfma<DT>::mma(a[t], opreg[t], t16);
        if (t + PD < NT) a[t + PD] = rd.read(0, t + PD);
      }
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        sX[wave][q4][lane] = (f32x4){t16[4 * q4], t16[4 * q4 + 1], t16[4 * q4 + 2], t16[4 * q4 + 3]};
    }
    // late waves: the next step's tile has landed (the one after may still
    // be in flight)
    if (late) wait_vm_steps<DMA_PER_STEP, NBUF - 2>(min(NBUF - 2, nsteps - 2 - step));
    // the pair's tiles are in LDS (the ring's DMA runs on across the barrier)
    barrier_lds_writes();
    if (active) {
      f32x16 sc, dp;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 x = sX[2 * qblk][q4][lane], y = sX[2 * qblk + 1][q4][lane];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          sc[4 * q4 + c] = x[c];
          dp[4 * q4 + c] = y[c];
        }
      }
      if constexpr (DROP) {
        // dP = D o (dO V^T): dropped elements 0, kept ones scaled
        dropout_row16(p, w.b, h, qi >> 2, (n0 + 4 * hh) >> 2, li & 3, p.drop_scale, dp);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[r] = fast_exp2(__builtin_fmaf(sc[r], sl2e, -lse2));
      // the causal mask only on steps that touch the diagonal (a wave-uniform
      // branch): key n0 + j is hidden from this lane's query while j > qk
      if (CAUSAL && n0 + KS - 1 > wq_lo_k) {
        const int qk = qi_k - n0;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (8 * (r >> 2) + 4 * hh + (r & 3) > qk) sc[r] = 0.f;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[r] = DROP ? sc[r] * (dp[r] - dlt) : sc[r] * dp[r];     // dS
      const u32x4 b0 = pack_operand<DT>(sc, 0), b1 = pack_operand<DT>(sc, 1);
      const TrReader<LK> trk(tk, lane);
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int cb = 0; cb < NCBH; ++cb)
        if (cb < nb) acc[cb] = Mfma<DT>::mma(trk.read(cb0 + cb, 0), b0, acc[cb]);
#pragma unroll
      for (int cb = 0; cb < NCBH; ++cb)
        if (cb < nb) acc[cb] = Mfma<DT>::mma(trk.read(cb0 + cb, 1), b1, acc[cb]);
      __builtin_amdgcn_s_setprio(0);
    }
  }
  if (!late) barrier_lds_writes();

  if (qvalid)
    store_dq<DT, ACC>(p, reinterpret_cast<uint16_t*>(p.dq) + qrow * qrs + (int64_t)h * p.d, cb0, hh, acc, nb);
}

// ----------------------------------------------------------------- dK / dV
// Head dims up to 128: 4 waves x 32 keys, 32 queries per step; the K and V
// operands of the wave's keys stay in registers for the whole workgroup.
// Each step DMAs the Q and dO tiles of one (query head, query tile) pair plus
// their LSE*log2(e) and -Delta vectors (one 4-byte DMA per wave: wave 0 LSE,
// wave 1 -Delta, other waves a dummy so that every wave issues the same
// number of DMAs and can use the same wait count).  Query rows past the real
// length arrive as zeros in Q, dO, LSE and Delta, so they add nothing.
// The tiles come through a ring of two buffers filled one step ahead, with
// one barrier per step.  The operand reads are pinned a fixed distance ahead
// of their MFMAs (scheduling barriers), since at 256 VGPRs the scheduler
// otherwise waits on each read just before its MFMA.
// ACC: add into dk / dv instead of writing them; DROP: dropout on the
// probabilities (the keep mask of dropout_block); PART: this workgroup takes
// kv_heads of the group's query heads and writes fp32 partial dK / dV planes
// (split GQA group); OCC: workgroups per CU the register budget is sized for;
// DE: the head dim rounded up to 16, the extent of the products.
template <int DT, int DPAD, bool CAUSAL, bool ACC, bool DROP, bool PART, int OCC, int DE>
__global__ __launch_bounds__(256, OCC) void dkdv_kernel(AttnParams p) {
  constexpr int NW = 4, BM = 32, NBUF = 2;
  constexpr int BN = 32 * NW;
  static_assert(BN == kKVTile, "the work lists are built for kKVTile keys per item");
  constexpr int NU = BM / 16;          // 16-query chunks per step
  static_assert(DE <= DPAD, "the products cover at most the padded head dim");
  constexpr int NT = (DE + 15) / 16;   // 16-wide k chunks of the products
  constexpr int NCB = (DE + 31) / 32;  // 32-column blocks of dK and dV
  using LQ = Lay<DPAD, true>;          // Q, dO: row reads (S, dP) and transposed reads (dK, dV)
  using Dma = TileDma<LQ, BM, NW>;
  constexpr int DMA_PER_STEP = 2 * Dma::PER_WAVE + 1;

  // ring of NBUF buffers of the Q and dO tiles and their LSE2 | Delta vectors
  __shared__ __attribute__((aligned(16))) uint16_t sQ[NBUF][LQ::template elems<BM>()];
  __shared__ __attribute__((aligned(16))) uint16_t sdO[NBUF][LQ::template elems<BM>()];
  __shared__ __attribute__((aligned(16))) float sVec[NBUF][2 * 64];
  __shared__ __attribute__((aligned(16))) uint16_t sSink[Dma::SINK ? 512 : 8];
  __shared__ __attribute__((aligned(16))) float sDummy[64];
  const int ntiles = uniform(p.hdr[kHdrNKVTiles]);
  int item, vh;
  xcd_split(blockIdx.x, PART ? p.hkv * p.kv_split : p.hkv, item, vh);
  if (item >= ntiles) return;
  // KV head g; with a split group, this workgroup's share of its query heads
  const int g = PART ? vh / p.kv_split : vh;
  const int sub = PART ? vh - g * p.kv_split : 0;
  const int ng = PART ? p.kv_heads : p.group;
  const WorkItem w = load_item(p.list, p.seq, item);
  const SeqInfo s = w.s;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, hh = lane >> 5;
  const int n0 = w.tile * BN;
  const int kj = n0 + wave * 32 + li;          // this lane's key (B-operand column)
  const int wk_lo = n0 + wave * 32, wk_hi = wk_lo + 31;
  // elements per row, and between consecutive tokens of a sequence
  const int64_t qrs = (int64_t)p.hq * p.d, kvrs = (int64_t)p.hkv * p.d;
  const int64_t qts = qrs * p.tsq, kvts = kvrs * p.tskv;
  const uint32_t q_rs_bytes = (uint32_t)(qts * 2);
  const int64_t kvoff = (int64_t)s.ok * kvrs + (int64_t)g * p.d;
  const uint16_t* kb = reinterpret_cast<const uint16_t*>(p.k) + kvoff;
  const uint16_t* vb = reinterpret_cast<const uint16_t*>(p.v) + kvoff;
  const u32x4 z4 = {0u, 0u, 0u, 0u};
  const float sl2e = p.scale_log2e;

  // query tiles that reach this key tile (query i sees key j iff
  // j <= i + diag), times the heads of the group
  const int diag = CAUSAL ? s.diag : 0;
  const int m_first = CAUSAL ? max(0, n0 - diag) / BM : 0;
  // the wave's keys and this lane's key shifted onto the query axis
  // (query i sees key j iff i >= j - diag)
  const int wk_lo_q = wk_lo - diag, wk_hi_q = wk_hi - diag, kj_q = kj - diag;
  const int m_last = (s.lq + BM - 1) / BM;
  const int nm = m_last > m_first ? m_last - m_first : 0;
  const int nsteps = nm * ng;
  const int h0 = g * p.group + sub * ng;
  // Steps walk the query tiles from the last one down, the group's heads
  // inside: key tiles of a sequence that start together then read the same
  // Q / dO tiles at the same time (from L2).  Two cursors follow that order
  // by increments (no division per step): the DMA's, NBUF-1 steps ahead, and
  // the compute loop's.

  Dma dma_q;
  dma_q.init(wave, lane, p.d, q_rs_bytes);
  // 4-byte DMA of the vector (LSE2 or Delta) rows i0 .. i0+BM-1 of head h
  const uint32_t vec_rs_bytes = (uint32_t)p.hq * (uint32_t)p.tsq * 4u;
  const uint32_t vec_voff = lane < BM ? (uint32_t)lane * vec_rs_bytes : kOutOfRange;
  // LDS byte addresses of ring buffer 0 (buffer b lies b buffer sizes on)
  const uint32_t lds_q = lds_addr(sQ[0]), lds_do = lds_addr(sdO[0]), lds_sink = lds_addr(sSink);
  const uint32_t lds_vec = wave == 0 ? lds_addr(sVec[0]) : (wave == 1 ? lds_addr(sVec[0]) + 256u : lds_addr(sDummy));
  const uint32_t vec_buf = wave < 2 ? (uint32_t)sizeof(sVec[0]) : 0u;
  const uint16_t* qg = reinterpret_cast<const uint16_t*>(p.q);
  const uint16_t* dog = reinterpret_cast<const uint16_t*>(p.dout);
  const float* vg = wave == 0 ? p.lse2 : p.delta;
  // DMA cursor: element offsets of the first row of (query tile, head) in
  // q / dout and in lse2 / delta, the head's index in the group, and the
  // tile's rows before the real end (>= 1 for every tile walked)
  const int64_t row_last = (int64_t)s.oq + (int64_t)(m_last - 1) * BM * p.tsq;
  int64_t dc_q = row_last * qrs + (int64_t)h0 * p.d;
  int64_t dc_v = row_last * p.hq + h0;
  int dc_hg = 0, dc_nrow = s.lq - (m_last - 1) * BM;
  // from the last head of a tile to the first head of the tile before it
  const int64_t q_back = (int64_t)BM * qts + (int64_t)(ng - 1) * p.d;
  const int64_t v_back = (int64_t)BM * p.tsq * p.hq + (ng - 1);
  auto issue = [&](int step) {
    const uint32_t buf = (uint32_t)(step % NBUF);
    const int nr = dc_nrow > BM ? BM : dc_nrow;
    dma_q.issue_rsrc(make_rsrc(qg + dc_q, (uint32_t)nr * q_rs_bytes), lds_q + buf * (uint32_t)sizeof(sQ[0]),
                     lds_sink, wave);
    dma_q.issue_rsrc(make_rsrc(dog + dc_q, (uint32_t)nr * q_rs_bytes), lds_do + buf * (uint32_t)sizeof(sdO[0]),
                     lds_sink, wave);
    dma<4>(make_rsrc(vg + dc_v, wave < 2 ? (uint32_t)nr * vec_rs_bytes : 0u), lds_vec + buf * vec_buf, vec_voff);
    if (++dc_hg == ng) {
      dc_hg = 0;
      dc_q -= q_back;
      dc_v -= v_back;
      dc_nrow += BM;
    } else {
      dc_q += p.d;
      dc_v += 1;
    }
  };
#pragma unroll
  for (int k = 0; k < NBUF - 1; ++k)
    if (k < nsteps) issue(k);

  // K and V operands of this wave's 32 keys (zero beyond the real keys)
  u32x4 kreg[NT], vreg[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int c = 16 * t + 8 * hh;
    const bool ok = kj < s.lk && c < p.d;
    kreg[t] = ok ? ldg16(kb + (int64_t)kj * kvts + c) : z4;
    vreg[t] = ok ? ldg16(vb + (int64_t)kj * kvts + c) : z4;
  }
  wait_vm<0>();

  f32x16 adk[NCB], adv[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    adk[cb] = zero16();
    adv[cb] = zero16();
  }

  // One barrier per step: the buffer refilled at step j (that of step j-1)
  // has been read by every wave once the wave passes step j's barrier.
  int cm = m_last - 1, chg = 0;   // compute cursor: query tile, head in the group
  for (int step = 0; step < nsteps; ++step) {
    // this step's tiles have landed
    wait_vm_steps<DMA_PER_STEP, NBUF - 2>(min(NBUF - 2, nsteps - 1 - step));
    barrier_lds_dma();
    if (step + NBUF - 1 < nsteps) issue(step + NBUF - 1);
    const int buf = step % NBUF;
    const uint32_t tq = lds_q + (uint32_t)buf * (uint32_t)sizeof(sQ[0]);
    const uint32_t tdo = lds_do + (uint32_t)buf * (uint32_t)sizeof(sdO[0]);
    const RowReader<LQ> rq(tq, lane), rdo(tdo, lane);
    const TrReader<LQ> trq(tq, lane), trdo(tdo, lane);
    const float* tvec = sVec[buf];
    const int i0 = cm * BM;
    const int h_step = h0 + chg;   // query head of this step
    if (++chg == ng) {
      chg = 0;
      --cm;
    }
    // waves with no real key, or whose keys all follow every query, idle
    if (wk_lo < s.lk && !(CAUSAL && i0 + BM - 1 < wk_lo_q)) {
      // S and dP interleaved, each Q / dO operand read two MFMAs ahead
      constexpr int PD = 2;
      u32x4 aq[NT], ado[NT];
      f32x16 sc = zero16(), dp;
      if constexpr (!DROP) {
        // dP accumulates onto -Delta of its rows, so the chain ends at dP - Delta
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 nd = *reinterpret_cast<const f32x4*>(&tvec[64 + 8 * q4 + 4 * hh]);
#pragma unroll
          for (int c = 0; c < 4; ++c) dp[4 * q4 + c] = nd[c];
        }
      } else {
        dp = zero16();
      }
#pragma unroll
      for (int t = 0; t < PD; ++t) {
        aq[t] = rq.read(0, t);
        ado[t] = rdo.read(0, t);
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        __builtin_amdgcn_sched_barrier(0);
        sc = Mfma<DT>::mma(aq[t], kreg[t], sc);
        if (t + PD < NT) aq[t + PD] = rq.read(0, t + PD);
        __builtin_amdgcn_sched_barrier(0);
        dp = Mfma<DT>::mma(ado[t], vreg[t], dp);
        if (t + PD < NT) ado[t + PD] = rdo.read(0, t + PD);
      }
      __builtin_amdgcn_sched_barrier(0);
      // P = exp2(S log2e - LSE log2e); the causal mask only on steps that
      // touch the diagonal (a wave-uniform branch): key kj is hidden from
      // query i0 + i while kj - diag > i0 + i
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(&tvec[8 * q4 + 4 * hh]);
#pragma unroll
        for (int c = 0; c < 4; ++c)
          sc[4 * q4 + c] = fast_exp2(__builtin_fmaf(sc[4 * q4 + c], sl2e, -l4[c]));
      }
      if (CAUSAL && i0 < wk_hi_q) {
        const int kq = kj_q - i0;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kq > 8 * (r >> 2) + 4 * hh + (r & 3)) sc[r] = 0.f;
      }
      // the key column of the 4 x 4 blocks at queries 8 q4 + 4 hh (+0..3):
      // this lane computes the Philox block of q4 = li & 3 (4 x 4: element
      // (i, j) is byte j & 3 of word i & 3); byte and quad transposes leave
      // in slot q4 this lane's key byte (j & 3 = li & 3) of that block's four
      // query rows, byte c for row c
      u32x4 mine;
      if constexpr (DROP)
        mine = quad_transpose(
            byte_transpose(dropout_block(p, w.b, h_step, ((i0 + 4 * hh) >> 2) + 2 * (li & 3), kj >> 2)), li & 3);
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(&tvec[64 + 8 * q4 + 4 * hh]);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int r = 4 * q4 + c;
          const float pr = sc[r];
          if constexpr (DROP) {
            // P o D for dV, and dS = P o (D o dP - Delta)
            const float dsc = keep_byte(mine[q4], c, p.drop_t) ? p.drop_scale : 0.f;
            sc[r] = pr * dsc;
            dp[r] = pr * __builtin_fmaf(dp[r], dsc, d4[c]);
          } else {
            dp[r] = pr * dp[r];
          }
        }
      }
      // P and dS as packed operands (the fp32 tiles die here)
      u32x4 bp[NU], bds[NU];
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        bp[u] = pack_operand<DT>(sc, u);
        bds[u] = pack_operand<DT>(dp, u);
      }
      // dV and dK interleaved, each transposed operand read one MFMA ahead
      constexpr int PDT = 1, NO = NU * NCB;
      u32x4 tdo[NO], tqo[NO];
#pragma unroll
      for (int o = 0; o < PDT; ++o) {
        tdo[o] = trdo.read(o % NCB, o / NCB);
        tqo[o] = trq.read(o % NCB, o / NCB);
      }
#pragma unroll
      for (int o = 0; o < NO; ++o) {
        const int u = o / NCB, cb = o % NCB;
        __builtin_amdgcn_sched_barrier(0);
        adv[cb] = Mfma<DT>::mma(tdo[o], bp[u], adv[cb]);
        if (o + PDT < NO) tdo[o + PDT] = trdo.read((o + PDT) % NCB, (o + PDT) / NCB);
        __builtin_amdgcn_sched_barrier(0);
        adk[cb] = Mfma<DT>::mma(tqo[o], bds[u], adk[cb]);
        if (o + PDT < NO) tqo[o + PDT] = trq.read((o + PDT) % NCB, (o + PDT) / NCB);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  if (kj < s.lk) {
    const int64_t row = (int64_t)kj * kvts;
    if constexpr (PART) {
      float* dkp = p.part + (int64_t)sub * p.part_plane + kvoff + row;
      store_dkdv_part(p, dkp, dkp + (int64_t)p.kv_split * p.part_plane, 0, hh, adk, adv);
    } else {
      store_dkdv<DT, ACC>(p, reinterpret_cast<uint16_t*>(p.dk) + kvoff + row,
                          reinterpret_cast<uint16_t*>(p.dv) + kvoff + row, 0, hh, adk, adv);
    }
  }
}

// ----------------------------------------------------------------- dK / dV, head dims 136..256
// At these head dims the fp32 dK and dV accumulators of 32 keys alone take
// 256 registers, which leaves no room for two waves per SIMD.  Here eight
// waves share 128 keys: waves 2 kb and 2 kb + 1 own key block kb (32 keys)
// and split the work by role.  Wave 2 kb holds K and accumulates dV: each
// step it forms S^T = K Q^T, P = exp(S - LSE) (masked), writes P to LDS and
// forms dV += P^T dO.  Wave 2 kb + 1 holds V and accumulates dK: it forms
// dP^T = V dO^T (onto -Delta), reads P back, forms dS = P o (dP - Delta) and
// dK += dS^T Q.  Each holds one full-width K or V operand and one full-width
// fp32 accumulator (128 registers at d = 256), P crosses LDS once, and the
// softmax and dS are each formed once per key block.  Two barriers per step:
// the ring's, and the one after P is written; waves 4..7 run half a step
// behind waves 0..3 (below).  Steps, cursors, masks, dropout and the split
// GQA group (PART) are those of dkdv_kernel with NW = 8, BM = 32; the DMA
// ring holds three buffers.  DE: the extent of the S / dP products (the head
// dim rounded up to 16).
template <int DT, bool CAUSAL, bool ACC, bool DROP, bool PART, int DE>
__global__ __launch_bounds__(512, 1) void dkdv_split_kernel(AttnParams p) {
  // Q / dO tiles 192 columns wide up to d = 192 (a quarter less DMA written
  // into LDS, which bounds this kernel), 256 above
  constexpr int DPAD = DE <= 192 ? 192 : 256, NW = 8, BM = 32, NBUF = 3;
  constexpr int BN = 16 * NW;          // keys per workgroup: NW / 2 blocks of 32
  static_assert(BN == kKVTile, "the work lists are built for kKVTile keys per item");
  static_assert(DE % 16 == 0 && DE > 128 && DE <= DPAD, "products over whole 16-wide k chunks");
  constexpr int NT = DE / 16;          // 16-wide k chunks of the S / dP products
  constexpr int NCB = (DE + 31) / 32;  // 32-column blocks of dK and dV
  constexpr int NU = BM / 16;          // 16-query chunks per step
  using LQ = Lay<DPAD, true>;          // Q, dO: row reads (S, dP) and transposed reads (dK, dV)
  using Dma = TileDma<LQ, BM, NW>;
  constexpr int DMA_PER_STEP = 2 * Dma::PER_WAVE + 1;

  __shared__ __attribute__((aligned(16))) uint16_t sQ[NBUF][LQ::template elems<BM>()];
  __shared__ __attribute__((aligned(16))) uint16_t sdO[NBUF][LQ::template elems<BM>()];
  __shared__ __attribute__((aligned(16))) float sVec[NBUF][2 * 64];
  __shared__ __attribute__((aligned(16))) uint16_t sSink[Dma::SINK ? 512 : 8];
  __shared__ __attribute__((aligned(16))) float sDummy[64];
  // P of each key block (written by the even wave for the odd one), as the
  // 16 accumulator registers of every lane: [key block][register / 4][lane]
  __shared__ __attribute__((aligned(16))) f32x4 sX[NW / 2][4][64];

  const int ntiles = uniform(p.hdr[kHdrNKVTiles]);
  int item, vh;
  xcd_split(blockIdx.x, PART ? p.hkv * p.kv_split : p.hkv, item, vh);
  if (item >= ntiles) return;
  // KV head g; with a split group, this workgroup's share of its query heads
  const int g = PART ? vh / p.kv_split : vh;
  const int sub = PART ? vh - g * p.kv_split : 0;
  const int ng = PART ? p.kv_heads : p.group;
  const WorkItem w = load_item(p.list, p.seq, item);
  const SeqInfo s = w.s;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // key block of this wave; odd: the V / dK wave of the block (even: K / dV)
  const int kblk = wave >> 1, odd = wave & 1;
  const int li = lane & 31, hh = lane >> 5;
  const int n0 = w.tile * BN;
  const int kj = n0 + kblk * 32 + li;          // this lane's key (B-operand column)
  const int wk_lo = n0 + kblk * 32, wk_hi = wk_lo + 31;
  const int64_t qrs = (int64_t)p.hq * p.d, kvrs = (int64_t)p.hkv * p.d;
  const int64_t qts = qrs * p.tsq, kvts = kvrs * p.tskv;
  const uint32_t q_rs_bytes = (uint32_t)(qts * 2);
  const int64_t kvoff = (int64_t)s.ok * kvrs + (int64_t)g * p.d;
  const u32x4 z4 = {0u, 0u, 0u, 0u};
  const float sl2e = p.scale_log2e;

  const int diag = CAUSAL ? s.diag : 0;
  const int m_first = CAUSAL ? max(0, n0 - diag) / BM : 0;
  const int wk_lo_q = wk_lo - diag, wk_hi_q = wk_hi - diag, kj_q = kj - diag;
  const int m_last = (s.lq + BM - 1) / BM;
  const int nm = m_last > m_first ? m_last - m_first : 0;
  const int nsteps = nm * ng;
  const int h0 = g * p.group + sub * ng;

  Dma dma_q;
  dma_q.init(wave, lane, p.d, q_rs_bytes);
  const uint32_t vec_rs_bytes = (uint32_t)p.hq * (uint32_t)p.tsq * 4u;
  const uint32_t vec_voff = lane < BM ? (uint32_t)lane * vec_rs_bytes : kOutOfRange;
  const uint32_t lds_q = lds_addr(sQ[0]), lds_do = lds_addr(sdO[0]), lds_sink = lds_addr(sSink);
  const uint32_t lds_vec = wave == 0 ? lds_addr(sVec[0]) : (wave == 1 ? lds_addr(sVec[0]) + 256u : lds_addr(sDummy));
  const uint32_t vec_buf = wave < 2 ? (uint32_t)sizeof(sVec[0]) : 0u;
  const uint16_t* qg = reinterpret_cast<const uint16_t*>(p.q);
  const uint16_t* dog = reinterpret_cast<const uint16_t*>(p.dout);
  const float* vg = wave == 0 ? p.lse2 : p.delta;
  const int64_t row_last = (int64_t)s.oq + (int64_t)(m_last - 1) * BM * p.tsq;
  int64_t dc_q = row_last * qrs + (int64_t)h0 * p.d;
  int64_t dc_v = row_last * p.hq + h0;
  int dc_hg = 0, dc_nrow = s.lq - (m_last - 1) * BM;
  const int64_t q_back = (int64_t)BM * qts + (int64_t)(ng - 1) * p.d;
  const int64_t v_back = (int64_t)BM * p.tsq * p.hq + (ng - 1);
  // DMA of the next tile in the cursor's order into ring buffer `buf`
  auto issue = [&](uint32_t buf) {
    const int nr = dc_nrow > BM ? BM : dc_nrow;
    dma_q.issue_rsrc(make_rsrc(qg + dc_q, (uint32_t)nr * q_rs_bytes), lds_q + buf * (uint32_t)sizeof(sQ[0]),
                     lds_sink, wave);
    dma_q.issue_rsrc(make_rsrc(dog + dc_q, (uint32_t)nr * q_rs_bytes), lds_do + buf * (uint32_t)sizeof(sdO[0]),
                     lds_sink, wave);
    dma<4>(make_rsrc(vg + dc_v, wave < 2 ? (uint32_t)nr * vec_rs_bytes : 0u), lds_vec + buf * vec_buf, vec_voff);
    if (++dc_hg == ng) {
      dc_hg = 0;
      dc_q -= q_back;
      dc_v -= v_back;
      dc_nrow += BM;
    } else {
      dc_q += p.d;
      dc_v += 1;
    }
  };
  // waves 4..7 run half a step behind waves 0..3 (see the loop)
  const int late = wave >= NW / 2 ? 1 : 0;
  for (int j = 0; j <= late; ++j)
    if (j < nsteps) issue((uint32_t)j);
  // ring buffer of the next tile this wave issues
  uint32_t ibuf = (uint32_t)late + 1u;

  // the full-width operand of this wave's product: K (even waves) or V (odd)
  const uint16_t* kvb = reinterpret_cast<const uint16_t*>(odd ? p.v : p.k) + kvoff;
  u32x4 kvreg[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int c = 16 * t + 8 * hh;
    kvreg[t] = (kj < s.lk && c < p.d) ? ldg16(kvb + (int64_t)kj * kvts + c) : z4;
  }
  wait_vm<0>();

  // dV (even waves) or dK (odd waves, unscaled) of this lane's key
  f32x16 ad[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) ad[cb] = zero16();

  // Waves 4..7 (key blocks 2, 3) run half a step behind waves 0..3: they
  // take one barrier before the loop (waves 0..3 one after it), so that a
  // late wave forms its tiles while the early wave on its SIMD (wave w - 4)
  // finishes its step, and finishes while that one forms the next step's
  // tiles: the softmax arithmetic of one runs under the products of the
  // other (in the same phase the matrix pipe idled through it).  Each wave
  // issues its share of a Q / dO tile's DMA at the start of its own step and
  // waits for it before the barrier that precedes the tile's first read: the
  // early waves tile step + 1 (first read after their next ring barrier),
  // the late waves tile step + 2 (after their P barrier of step + 1).
  // A tile is read until the late waves' ring barrier of the next step,
  // hence a ring of three.
  if (late) {
    wait_vm_steps<DMA_PER_STEP, NBUF - 2>(min(NBUF - 2, nsteps - 1));
    barrier_lds_writes();
  }
  int cm = m_last - 1, chg = 0;
  for (int step = 0; step < nsteps; ++step) {
    // early waves: this step's tile has landed; late waves: the early waves'
    // P tiles are in LDS
    if (!late) wait_vm<0>();
    barrier_lds_writes();
    if (step + 1 + late < nsteps) issue(ibuf);
    ibuf = ibuf == NBUF - 1 ? 0u : ibuf + 1u;
    const int buf = step % NBUF;
    const uint32_t tq = lds_q + (uint32_t)buf * (uint32_t)sizeof(sQ[0]);
    const uint32_t tdo = lds_do + (uint32_t)buf * (uint32_t)sizeof(sdO[0]);
    const float* tvec = sVec[buf];
    const int i0 = cm * BM;
    const int h_step = h0 + chg;
    if (++chg == ng) {
      chg = 0;
      --cm;
    }
    // both waves of a key block are active or idle together
    const bool active = wk_lo < s.lk && !(CAUSAL && i0 + BM - 1 < wk_lo_q);
    f32x16 acc;   // S^T, then P (even waves); dP^T onto -Delta (odd waves)
    if (active) {
      // operands read two MFMAs ahead
      constexpr int PD = 2;
      const RowReader<LQ> rd(odd ? tdo : tq, lane);
      if (odd && !DROP) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 nd = *reinterpret_cast<const f32x4*>(&tvec[64 + 8 * q4 + 4 * hh]);
#pragma unroll
          for (int c = 0; c < 4; ++c) acc[4 * q4 + c] = nd[c];
        }
      } else {
        acc = zero16();
      }
      u32x4 a[NT];
#pragma unroll
      for (int t = 0; t < PD; ++t) a[t] = rd.read(0, t);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        __builtin_amdgcn_sched_barrier(0);
        acc = Mfma<DT>::mma(a[t], kvreg[t], acc);
        if (t + PD < NT) a[t + PD] = rd.read(0, t + PD);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (!odd) {
        // P, masked, for both waves of the key block
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(&tvec[8 * q4 + 4 * hh]);
#pragma unroll
          for (int c = 0; c < 4; ++c)
            acc[4 * q4 + c] = fast_exp2(__builtin_fmaf(acc[4 * q4 + c], sl2e, -l4[c]));
        }
        if (CAUSAL && i0 < wk_hi_q) {
          const int kq = kj_q - i0;
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (kq > 8 * (r >> 2) + 4 * hh + (r & 3)) acc[r] = 0.f;
        }
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          sX[kblk][q4][lane] = (f32x4){acc[4 * q4], acc[4 * q4 + 1], acc[4 * q4 + 2], acc[4 * q4 + 3]};
      }
    }
    // late waves: the next step's tile has landed (the one after may still
    // be in flight)
    if (late) wait_vm_steps<DMA_PER_STEP, NBUF - 2>(min(NBUF - 2, nsteps - 2 - step));
    // P is in LDS (the ring's DMA runs on across the barrier)
    barrier_lds_writes();
    if (active) {
      u32x4 mine;
      if constexpr (DROP)
        mine = quad_transpose(
            byte_transpose(dropout_block(p, w.b, h_step, ((i0 + 4 * hh) >> 2) + 2 * (li & 3), kj >> 2)), li & 3);
      if (!odd) {
        // (P o D) for dV: dropped values 0, kept ones scaled
        if constexpr (DROP) {
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const int r = 4 * q4 + c;
              acc[r] = acc[r] * (keep_byte(mine[q4], c, p.drop_t) ? p.drop_scale : 0.f);
            }
        }
      } else {
        // dS = P o (dP - Delta), with dropout P o (D o dP - Delta)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 pr = sX[kblk][q4][lane];
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(&tvec[64 + 8 * q4 + 4 * hh]);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int r = 4 * q4 + c;
            if constexpr (DROP) {
              const float dsc = keep_byte(mine[q4], c, p.drop_t) ? p.drop_scale : 0.f;
              acc[r] = pr[c] * __builtin_fmaf(acc[r], dsc, d4[c]);
            } else {
              acc[r] = pr[c] * acc[r];
            }
          }
        }
      }
      u32x4 b[NU];
#pragma unroll
      for (int u = 0; u < NU; ++u) b[u] = pack_operand<DT>(acc, u);
      // dV += (P o D)^T dO or dK += dS^T Q over every column block, the
      // transposed operand read two MFMAs ahead
      const TrReader<LQ> tr(odd ? tq : tdo, lane);
      constexpr int PT = 2, NO = NU * NCB;
      u32x4 to[NO];
#pragma unroll
      for (int o = 0; o < PT; ++o) to[o] = tr.read(o % NCB, o / NCB);
#pragma unroll
      for (int o = 0; o < NO; ++o) {
        __builtin_amdgcn_sched_barrier(0);
        ad[o % NCB] = Mfma<DT>::mma(to[o], b[o / NCB], ad[o % NCB]);
        if (o + PT < NO) to[o + PT] = tr.read((o + PT) % NCB, (o + PT) / NCB);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if (!late) barrier_lds_writes();

  if (kj < s.lk) {
    const int64_t row = (int64_t)kj * kvts;
    if constexpr (PART) {
      // the dK planes, then the dV planes (unscaled)
      float* dkp = p.part + (int64_t)sub * p.part_plane + kvoff + row;
      store_row_part(p, odd ? dkp : dkp + (int64_t)p.kv_split * p.part_plane, hh, ad);
    } else {
      uint16_t* out = reinterpret_cast<uint16_t*>(odd ? p.dk : p.dv) + kvoff + row;
      store_row<DT, ACC>(p, out, 0, hh, ad, odd ? p.scale : 1.f);
    }
  }
}

// ----------------------------------------------------------------- split GQA group: the sum
// Sums the kv_split partial dK and dV planes of every key row of a work item
// in plane order (fixed, so the result is bitwise repeatable), scales dK,
// rounds once and writes dk / dv (ACC: adds into them).  One workgroup per
// (key tile, KV head) of the dK/dV work list; rows past the real length are
// left to the zero fill, as in the dK/dV kernels.
template <int DT, bool ACC>
__global__ __launch_bounds__(256) void dkdv_reduce_kernel(AttnParams p) {
  const int ntiles = uniform(p.hdr[kHdrNKVTiles]);
  const int item = blockIdx.x / p.hkv, g = blockIdx.x - item * p.hkv;
  if (item >= ntiles) return;
  const WorkItem w = load_item(p.list, p.seq, item);
  const SeqInfo s = w.s;
  const int64_t kvrs = (int64_t)p.hkv * p.d, kvts = kvrs * p.tskv;
  const int64_t kvoff = (int64_t)s.ok * kvrs + (int64_t)g * p.d;
  const int n0 = w.tile * kKVTile;
  const int rows = min(kKVTile, s.lk - n0);
  const int chunks = p.d >> 2;   // 4-column pieces per row
  const int64_t plane = p.part_plane;
  const float* dvp = p.part + (int64_t)p.kv_split * plane;
  for (int i = threadIdx.x; i < rows * chunks; i += 256) {
    const int r = i / chunks, c = 4 * (i - r * chunks);
    const int64_t off = kvoff + (int64_t)(n0 + r) * kvts + c;
    f32x4 sk = *reinterpret_cast<const f32x4*>(p.part + off);
    f32x4 sv = *reinterpret_cast<const f32x4*>(dvp + off);
    for (int j = 1; j < p.kv_split; ++j) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(p.part + j * plane + off);
      const f32x4 b = *reinterpret_cast<const f32x4*>(dvp + j * plane + off);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sk[e] += a[e];
        sv[e] += b[e];
      }
    }
    float xk[4], xv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      xk[e] = sk[e] * p.scale;
      xv[e] = sv[e];
    }
    uint16_t* dkb = reinterpret_cast<uint16_t*>(p.dk) + off;
    uint16_t* dvb = reinterpret_cast<uint16_t*>(p.dv) + off;
    if constexpr (ACC) {
      add_stored<DT>(xk, *reinterpret_cast<const u32x2*>(dkb));
      add_stored<DT>(xv, *reinterpret_cast<const u32x2*>(dvb));
    }
    *reinterpret_cast<u32x2*>(dkb) = (u32x2){Mfma<DT>::pack2(xk[0], xk[1]), Mfma<DT>::pack2(xk[2], xk[3])};
    *reinterpret_cast<u32x2*>(dvb) = (u32x2){Mfma<DT>::pack2(xv[0], xv[1]), Mfma<DT>::pack2(xv[2], xv[3])};
  }
}

// ----------------------------------------------------------------- launchers
// dropout is not combined with accumulation (the chunked entry points take none)
// DE: the extent of the products, the head dim rounded up to 16 (the split
// dK/dV takes its column blocks in pairs); the k chunks and column blocks
// past it hold no real column
template <int DT, int DPAD, bool CAUSAL, int DE>
static void launch_dq_c(const AttnParams& p, int grid, hipStream_t st) {
  const dim3 g(grid), blk(256);
  if (p.accumulate & kAccDq) hipLaunchKernelGGL((dq_kernel<DT, DPAD, CAUSAL, true, false, DE>), g, blk, 0, st, p);
  else if (p.drop_t) hipLaunchKernelGGL((dq_kernel<DT, DPAD, CAUSAL, false, true, DE>), g, blk, 0, st, p);
  else hipLaunchKernelGGL((dq_kernel<DT, DPAD, CAUSAL, false, false, DE>), g, blk, 0, st, p);
}

template <int DT, bool CAUSAL, int DE>
static void launch_dq_split_c(const AttnParams& p, int grid, hipStream_t st) {
  const dim3 g(grid), blk(512);
  if (p.accumulate & kAccDq) hipLaunchKernelGGL((dq_split_kernel<DT, CAUSAL, true, false, DE>), g, blk, 0, st, p);
  else if (p.drop_t) hipLaunchKernelGGL((dq_split_kernel<DT, CAUSAL, false, true, DE>), g, blk, 0, st, p);
  else hipLaunchKernelGGL((dq_split_kernel<DT, CAUSAL, false, false, DE>), g, blk, 0, st, p);
}

template <int DT, int DE>
static void launch_dq_split_d(const AttnParams& p, bool causal, int grid, hipStream_t st) {
  if (causal) launch_dq_split_c<DT, true, DE>(p, grid, st);
  else launch_dq_split_c<DT, false, DE>(p, grid, st);
}

template <int DT>
static void launch_dq_split(const AttnParams& p, bool causal, int grid, hipStream_t st) {
  switch ((p.d + 15) >> 4) {
    case 13: launch_dq_split_d<DT, 208>(p, causal, grid, st); break;
    case 14: launch_dq_split_d<DT, 224>(p, causal, grid, st); break;
    case 15: launch_dq_split_d<DT, 240>(p, causal, grid, st); break;
    default: launch_dq_split_d<DT, 256>(p, causal, grid, st);
  }
}

template <int DT, int DPAD, int DE>
static void launch_dq_d(const AttnParams& p, bool causal, int grid, hipStream_t st) {
  if (causal) launch_dq_c<DT, DPAD, true, DE>(p, grid, st);
  else launch_dq_c<DT, DPAD, false, DE>(p, grid, st);
}

template <int DT>
static void launch_dq_dt(const AttnParams& p, bool causal, int grid, hipStream_t st) {
  switch ((p.d + 15) >> 4) {
    case 1: case 2: launch_dq_d<DT, 32, 32>(p, causal, grid, st); break;
    case 3: launch_dq_d<DT, 64, 48>(p, causal, grid, st); break;
    case 4: launch_dq_d<DT, 64, 64>(p, causal, grid, st); break;
    case 5: launch_dq_d<DT, 128, 80>(p, causal, grid, st); break;
    case 6: launch_dq_d<DT, 128, 96>(p, causal, grid, st); break;
    case 7: launch_dq_d<DT, 128, 112>(p, causal, grid, st); break;
    case 8: launch_dq_d<DT, 128, 128>(p, causal, grid, st); break;
    // head dims 136..192 on 192-wide tiles (above, Q, dO and the dQ
    // accumulator outgrow the registers: the split kernel)
    case 9: launch_dq_d<DT, 192, 144>(p, causal, grid, st); break;
    case 10: launch_dq_d<DT, 192, 160>(p, causal, grid, st); break;
    case 11: launch_dq_d<DT, 192, 176>(p, causal, grid, st); break;
    case 12: launch_dq_d<DT, 192, 192>(p, causal, grid, st); break;
    default: launch_dq_split<DT>(p, causal, grid, st);
  }
}

hipError_t launch_dq(const AttnParams& p, int dtype, bool causal, int max_q_tiles, hipStream_t st) {
  const int grid = max_q_tiles * p.hq;
  if (grid <= 0) return hipSuccess;
  if (dtype == kBF16) launch_dq_dt<kBF16>(p, causal, grid, st);
  else launch_dq_dt<kFP16>(p, causal, grid, st);
  return hipGetLastError();
}

// keys per dK/dV work item for a head dim
int dkdv_tile(int d) { (void)d; return kKVTile; }

hipError_t launch_dkdv_reduce(const AttnParams& p, int dtype, int max_kv_tiles, hipStream_t st) {
  const int grid = max_kv_tiles * p.hkv;
  if (grid <= 0) return hipSuccess;
  const bool acc = p.accumulate & kAccDkDv;
  if (dtype == kBF16) {
    if (acc) hipLaunchKernelGGL((dkdv_reduce_kernel<kBF16, true>), dim3(grid), dim3(256), 0, st, p);
    else hipLaunchKernelGGL((dkdv_reduce_kernel<kBF16, false>), dim3(grid), dim3(256), 0, st, p);
  } else {
    if (acc) hipLaunchKernelGGL((dkdv_reduce_kernel<kFP16, true>), dim3(grid), dim3(256), 0, st, p);
    else hipLaunchKernelGGL((dkdv_reduce_kernel<kFP16, false>), dim3(grid), dim3(256), 0, st, p);
  }
  return hipGetLastError();
}

template <int DT, bool CAUSAL, int DE>
static void launch_dkdv_split_c(const AttnParams& p, int grid, hipStream_t st) {
  const dim3 g(grid), blk(512);
  if (p.kv_split > 1) {
    if (p.drop_t) hipLaunchKernelGGL((dkdv_split_kernel<DT, CAUSAL, false, true, true, DE>), g, blk, 0, st, p);
    else hipLaunchKernelGGL((dkdv_split_kernel<DT, CAUSAL, false, false, true, DE>), g, blk, 0, st, p);
  } else if (p.accumulate & kAccDkDv)
    hipLaunchKernelGGL((dkdv_split_kernel<DT, CAUSAL, true, false, false, DE>), g, blk, 0, st, p);
  else if (p.drop_t) hipLaunchKernelGGL((dkdv_split_kernel<DT, CAUSAL, false, true, false, DE>), g, blk, 0, st, p);
  else hipLaunchKernelGGL((dkdv_split_kernel<DT, CAUSAL, false, false, false, DE>), g, blk, 0, st, p);
}

template <int DT, int DE>
static void launch_dkdv_split_d(const AttnParams& p, bool causal, int grid, hipStream_t st) {
  if (causal) launch_dkdv_split_c<DT, true, DE>(p, grid, st);
  else launch_dkdv_split_c<DT, false, DE>(p, grid, st);
}

template <int DT>
static void launch_dkdv_split(const AttnParams& p, bool causal, int grid, hipStream_t st) {
  switch ((p.d + 15) >> 4) {
    case 9: launch_dkdv_split_d<DT, 144>(p, causal, grid, st); break;
    case 10: launch_dkdv_split_d<DT, 160>(p, causal, grid, st); break;
    case 11: launch_dkdv_split_d<DT, 176>(p, causal, grid, st); break;
    case 12: launch_dkdv_split_d<DT, 192>(p, causal, grid, st); break;
    case 13: launch_dkdv_split_d<DT, 208>(p, causal, grid, st); break;
    case 14: launch_dkdv_split_d<DT, 224>(p, causal, grid, st); break;
    case 15: launch_dkdv_split_d<DT, 240>(p, causal, grid, st); break;
    default: launch_dkdv_split_d<DT, 256>(p, causal, grid, st);
  }
}

// a split group writes partial planes; dropout and accumulation then act in
// the kernel and in the sum respectively
template <int DT, int DPAD, bool CAUSAL, int OCC, int DE>
static void launch_dkdv_c(const AttnParams& p, int grid, hipStream_t st) {
  const dim3 g(grid), blk(256);
  if (p.kv_split > 1) {
    if (p.drop_t)
      hipLaunchKernelGGL((dkdv_kernel<DT, DPAD, CAUSAL, false, true, true, OCC, DE>), g, blk, 0, st, p);
    else
      hipLaunchKernelGGL((dkdv_kernel<DT, DPAD, CAUSAL, false, false, true, OCC, DE>), g, blk, 0, st, p);
  } else if (p.accumulate & kAccDkDv)
    hipLaunchKernelGGL((dkdv_kernel<DT, DPAD, CAUSAL, true, false, false, OCC, DE>), g, blk, 0, st, p);
  else if (p.drop_t)
    hipLaunchKernelGGL((dkdv_kernel<DT, DPAD, CAUSAL, false, true, false, OCC, DE>), g, blk, 0, st, p);
  else
    hipLaunchKernelGGL((dkdv_kernel<DT, DPAD, CAUSAL, false, false, false, OCC, DE>), g, blk, 0, st, p);
}

template <int DT, int DPAD, int OCC, int DE>
static void launch_dkdv_d(const AttnParams& p, bool causal, int grid, hipStream_t st) {
  if (causal) launch_dkdv_c<DT, DPAD, true, OCC, DE>(p, grid, st);
  else launch_dkdv_c<DT, DPAD, false, OCC, DE>(p, grid, st);
}

template <int DT>
static void launch_dkdv_dt(const AttnParams& p, bool causal, int grid, hipStream_t st) {
  // three workgroups per CU up to d = 64 (<= 168 VGPRs), two at 128
  switch ((p.d + 15) >> 4) {
    case 1: case 2: launch_dkdv_d<DT, 32, 3, 32>(p, causal, grid, st); break;
    case 3: launch_dkdv_d<DT, 64, 3, 48>(p, causal, grid, st); break;
    case 4: launch_dkdv_d<DT, 64, 3, 64>(p, causal, grid, st); break;
    case 5: launch_dkdv_d<DT, 128, 2, 80>(p, causal, grid, st); break;
    case 6: launch_dkdv_d<DT, 128, 2, 96>(p, causal, grid, st); break;
    case 7: launch_dkdv_d<DT, 128, 2, 112>(p, causal, grid, st); break;
    case 8: launch_dkdv_d<DT, 128, 2, 128>(p, causal, grid, st); break;
    default: launch_dkdv_split<DT>(p, causal, grid, st);
  }
}

hipError_t launch_dkdv(const AttnParams& p, int dtype, bool causal, int max_kv_tiles, hipStream_t st) {
  const int grid = max_kv_tiles * p.hkv * p.kv_split;
  if (grid <= 0) return hipSuccess;
  if (dtype == kBF16) launch_dkdv_dt<kBF16>(p, causal, grid, st);
  else launch_dkdv_dt<kFP16>(p, causal, grid, st);
  return hipGetLastError();
}

}  // namespace attn
