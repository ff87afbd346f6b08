// Varlen tile scheduler and uncovered-row zero fill.
//
// The scheduler turns the four cu_seqlens arrays into (a) a per-sequence
// table of padded offsets and real lengths and (b) work lists of
// (sequence, tile) for the compute kernels.  Real boundaries mask, padded
// boundaries index (TransformerEngine issue 2892, "Expected Behavior").
// Sequences without a real query or without a real key get no tile: their
// rows are written by the zero fill, which also covers padding rows and rows
// outside every slot (issue 2448, "Expected behavior": KV of a sequence with
// no valid query must come back as zeros).  Tiles are grouped by sequence,
// heaviest sequence first and heaviest tile first within it, so that the long
// causal tiles start early and a sequence's tiles run together.
#include "common.h"

namespace attn {

constexpr int kSchedThreads = 1024;

// ceil(a / b) for a >= 0, b > 0
__device__ __forceinline__ int cdiv(int a, int b) { return (a + b - 1) / b; }

// Work key of a query tile: keys it visits, in 64-key units.  causal: 0 no
// triangle, 1 top-left, 2 bottom-right (query i sees key j iff
// j <= i + causal_diag).
__device__ __forceinline__ int q_tile_key(const SeqInfo& s, int m, int tile, int causal) {
  int hi = min(s.lq, (m + 1) * tile);
  int keys = causal ? max(0, min(s.lk, hi + s.diag)) : s.lk;
  return min(cdiv(keys, 64), kSchedKeys - 1);
}

// Work key of a key tile: queries that reach it, in 64-query units.
__device__ __forceinline__ int kv_tile_key(const SeqInfo& s, int n, int tile, int causal) {
  int q = causal ? max(0, s.lq - max(0, n * tile - s.diag)) : s.lq;
  return min(cdiv(q, 64), kSchedKeys - 1);
}

// Work key of a sequence's key tiles: that of its first tile, the heaviest
// (the queries that reach key tile n never grow with n).
__device__ __forceinline__ int seq_kv_key(const SeqInfo& s, int tile, int causal) {
  return kv_tile_key(s, 0, tile, causal);
}

// Work key of a sequence's n query tiles: that of its last, the heaviest.
__device__ __forceinline__ int seq_q_key(const SeqInfo& s, int n, int tile, int causal) {
  return q_tile_key(s, n - 1, tile, causal);
}

// Exclusive prefix over hist[] in DESCENDING key order, in place:
// hist[k] becomes the number of tiles with a larger key.  Returns the total.
__device__ int scan_desc(int* hist, int* part) {
  const int tid = threadIdx.x;
  constexpr int per = kSchedKeys / kSchedThreads;  // keys per thread
  // thread tid owns descending positions [tid*per, tid*per+per)
  int loc[per];
  int sum = 0;
#pragma unroll
  for (int i = 0; i < per; ++i) {
    loc[i] = hist[kSchedKeys - 1 - (tid * per + i)];
    sum += loc[i];
  }
  part[tid] = sum;
  __syncthreads();
  // Hillis-Steele inclusive scan over the per-thread sums
  for (int off = 1; off < kSchedThreads; off <<= 1) {
    int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = part[tid] - sum;
  const int total = part[kSchedThreads - 1];
#pragma unroll
  for (int i = 0; i < per; ++i) {
    hist[kSchedKeys - 1 - (tid * per + i)] = run;
    run += loc[i];
  }
  __syncthreads();
  return total;
}

// Builds one list.  kv_side selects which length is tiled.  The order of
// items with equal keys depends on LDS atomics and is not fixed; every output
// element is produced by exactly one work item with a fixed internal order,
// so results do not depend on the list order.
//
// Tiles are listed by sequence, the sequence with the heaviest tile first,
// each sequence's tiles contiguous and heaviest first: the tiles of a
// sequence then run together and read the other side's tiles in step
// (shared in L2).
__device__ int build_list(const SchedParams& p, bool kv_side, int tile, int2* list, int* hist,
                          int* part) {
  const int tid = threadIdx.x;
  for (int k = tid; k < kSchedKeys; k += kSchedThreads) hist[k] = 0;
  __syncthreads();
  for (int b = tid; b < p.batch; b += kSchedThreads) {
    SeqInfo s = p.seq[b];
    if (s.lq == 0 || s.lk == 0) continue;
    const int n = cdiv(kv_side ? s.lk : s.lq, tile);
    atomicAdd(&hist[kv_side ? seq_kv_key(s, tile, p.causal) : seq_q_key(s, n, tile, p.causal)], n);
  }
  __syncthreads();
  const int total = scan_desc(hist, part);
  for (int b = tid; b < p.batch; b += kSchedThreads) {
    SeqInfo s = p.seq[b];
    if (s.lq == 0 || s.lk == 0) continue;
    const int n = cdiv(kv_side ? s.lk : s.lq, tile);
    const int pos =
        atomicAdd(&hist[kv_side ? seq_kv_key(s, tile, p.causal) : seq_q_key(s, n, tile, p.causal)], n);
    // tiles in decreasing work: causal key tiles are reached by fewer queries
    // the later they sit, causal query tiles see more keys
    for (int t = 0; t < n; ++t) list[pos + t] = make_int2(b, kv_side ? t : n - 1 - t);
  }
  __syncthreads();
  return total;
}

__global__ __launch_bounds__(kSchedThreads) void sched_kernel(SchedParams p) {
  __shared__ int hist[kSchedKeys];
  __shared__ int part[kSchedThreads];
  __shared__ int s_bad;
  const int tid = threadIdx.x;
  if (tid == 0) s_bad = 0;
  __syncthreads();
  const bool thd = p.layout == kLayoutThd;
  const int32_t* cqp = p.cu_qp ? p.cu_qp : p.cu_q;
  const int32_t* ckp = p.cu_kp ? p.cu_kp : p.cu_kv;
  for (int b = tid; b < p.batch; b += kSchedThreads) {
    // batched layouts: a missing real-length array means full slots
    const int64_t lq = p.cu_q ? (int64_t)p.cu_q[b + 1] - p.cu_q[b] : p.slot_q;
    const int64_t lk = p.cu_kv ? (int64_t)p.cu_kv[b + 1] - p.cu_kv[b] : p.slot_kv;
    // slot [pq0, pq1) in token positions (rows for THD and bshd; sbhd
    // slots are strided, their first row is b)
    int64_t pq0, pq1, pk0, pk1;
    if (thd) {
      pq0 = cqp[b]; pq1 = cqp[b + 1]; pk0 = ckp[b]; pk1 = ckp[b + 1];
    } else {
      pq0 = (int64_t)b * p.slot_q; pq1 = pq0 + p.slot_q;
      pk0 = (int64_t)b * p.slot_kv; pk1 = pk0 + p.slot_kv;
    }
    // real length within [0, slot]; slot within [0, total]: with every b
    // checked this also makes the padded arrays non-decreasing, so slots are
    // disjoint.
    const bool bad = lq < 0 || lq > pq1 - pq0 || lk < 0 || lk > pk1 - pk0 || pq0 < 0 ||
                     pq1 > p.total_q || pk0 < 0 || pk1 > p.total_kv;
    if (bad) atomicOr(&s_bad, 1);
    const bool sbhd = p.layout == kLayoutSbhd;
    SeqInfo s;
    s.oq = bad ? 0 : (sbhd ? b : (int)pq0);
    s.lq = bad ? 0 : (int)lq;
    s.ok = bad ? 0 : (sbhd ? b : (int)pk0);
    s.lk = bad ? 0 : (int)lk;
    // causal diagonal: top-left 0 (or the chunk positions' difference),
    // bottom-right Lk - Lq; clamped to [-Lq, Lk], which leaves the mask as
    // it is (beyond those bounds every key, or no key, is visible)
    int64_t diag = 0;
    if (p.causal == 2) diag = lk - lq;
    else if (p.causal == 1)
      diag = (int64_t)(p.q_pos0 ? p.q_pos0[b] : 0) - (int64_t)(p.kv_pos0 ? p.kv_pos0[b] : 0);
    s.diag = bad ? 0 : (int)(diag < -lq ? -lq : (diag > lk ? lk : diag));
    p.seq[b] = s;
  }
  __syncthreads();
  const int bad = s_bad;
  int nq = 0, nk = 0;
  if (!bad) {
    __threadfence_block();
    if (p.q_tile > 0) nq = build_list(p, false, p.q_tile, p.q_list, hist, part);
    if (p.kv_tile > 0) nk = build_list(p, true, p.kv_tile, p.kv_list, hist, part);
  }
  if (tid == 0) {
    p.hdr[kHdrStatus] = bad ? 1 : 0;
    p.hdr[kHdrNQTiles] = nq;
    p.hdr[kHdrNKVTiles] = nk;
  }
}

// ----------------------------------------------------------------- zero fill
// One workgroup per 64 rows.  A query row is covered when it lies inside the
// real part of a sequence that has at least one real key; a key row when it
// lies inside the real part of a sequence with at least one real query.
// Uncovered rows get +0.0 (and lse = -inf).  With bad cu_seqlens data no row
// is covered.
constexpr int kZeroRows = 64;

__global__ __launch_bounds__(256) void zero_fill_kernel(ZeroParams p) {
  __shared__ int s_uncov[kZeroRows];
  __shared__ int s_n;
  const int tid = threadIdx.x;
  const int row0 = blockIdx.x * kZeroRows;
  if (tid == 0) s_n = 0;
  __syncthreads();
  if (tid < kZeroRows && row0 + tid < p.rows) {
    const int t = row0 + tid;
    bool cov = false;
    if (p.hdr[kHdrStatus] == 0 && p.batch > 0 && p.layout != kLayoutThd) {
      // batched layouts: row t is token i of sequence b
      const bool sbhd = p.layout == kLayoutSbhd;
      const int b = sbhd ? t % p.batch : t / p.slot;
      const int i = sbhd ? t / p.batch : t % p.slot;
      if (b < p.batch) {
        SeqInfo s = p.seq[b];
        cov = p.kv_side ? (i < s.lk && s.lq > 0) : (i < s.lq && s.lk > 0);
      }
    } else if (p.hdr[kHdrStatus] == 0 && p.batch > 0) {
      // largest b with offset(b) <= t (offsets are non-decreasing when valid)
      int lo = 0, hi = p.batch - 1, b = -1;
      while (lo <= hi) {
        int mid = (lo + hi) >> 1;
        int off = p.kv_side ? p.seq[mid].ok : p.seq[mid].oq;
        if (off <= t) { b = mid; lo = mid + 1; } else { hi = mid - 1; }
      }
      if (b >= 0) {
        SeqInfo s = p.seq[b];
        cov = p.kv_side ? (t - s.ok < s.lk && s.lq > 0) : (t - s.oq < s.lq && s.lk > 0);
      }
    }
    if (!cov) {
      int slot = atomicAdd(&s_n, 1);
      s_uncov[slot] = t;
    }
  }
  __syncthreads();
  const int n = s_n;
  const int chunks = p.width >> 3;   // 16-byte chunks per row (width % 8 == 0)
  const u32x4 z = {0u, 0u, 0u, 0u};
  for (int i = 0; i < n; ++i) {
    const int64_t t = s_uncov[i];
    for (int c = tid; c < chunks; c += 256) {
      if (p.t0) reinterpret_cast<u32x4*>(p.t0)[t * chunks + c] = z;
      if (p.t1) reinterpret_cast<u32x4*>(p.t1)[t * chunks + c] = z;
    }
    if (p.lse)
      for (int h = tid; h < p.lse_heads; h += 256) p.lse[t * p.lse_heads + h] = -__builtin_inff();
  }
}

// ----------------------------------------------------------------- launchers
hipError_t launch_sched(const SchedParams& p, hipStream_t st) {
  hipLaunchKernelGGL(sched_kernel, dim3(1), dim3(kSchedThreads), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_zero_fill(const ZeroParams& p, hipStream_t st) {
  if (p.rows <= 0) return hipSuccess;
  const int blocks = (p.rows + kZeroRows - 1) / kZeroRows;
  hipLaunchKernelGGL(zero_fill_kernel, dim3(blocks), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace attn
