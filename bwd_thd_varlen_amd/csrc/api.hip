// Host side of the C ABI declared in include/attn_thd.h: argument checks,
// workspace layout and the launch sequence on the caller's stream.  Nothing
// here allocates device memory, synchronises or keeps state between calls.
#include <atomic>
#include <cmath>
#include <cstddef>
#include <cstdint>

#include "../../include/attn_thd.h"
#include "common.h"

static_assert(ATTN_THD_ACC_DQ == attn::kAccDq && ATTN_THD_ACC_DKDV == attn::kAccDkDv,
              "accumulate bits of the header and the kernels agree");

namespace attn {
hipError_t launch_sched(const SchedParams& p, hipStream_t st);
hipError_t launch_zero_fill(const ZeroParams& p, hipStream_t st);
hipError_t launch_fwd(const AttnParams& p, int dtype, bool causal, int max_q_tiles, hipStream_t st);
hipError_t launch_dq(const AttnParams& p, int dtype, bool causal, int max_q_tiles, hipStream_t st);
hipError_t launch_dkdv(const AttnParams& p, int dtype, bool causal, int max_kv_tiles, hipStream_t st);
hipError_t launch_dkdv_reduce(const AttnParams& p, int dtype, int max_kv_tiles, hipStream_t st);
hipError_t launch_merge(void* out, float* lse, const void* out_part, const float* lse_part,
                        int64_t rows, int d, int dtype, hipStream_t st);
hipError_t launch_decode_e4m3(const void* src, void* dst, int64_t n, int dtype, hipStream_t st);
int dkdv_tile(int d);
}  // namespace attn

namespace {

using namespace attn;

constexpr size_t kAlign = 256;

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// the kernels move rows in 16-byte pieces
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Layout {
  size_t hdr, seq, q_list, kv_list, delta, lse2, part, total;
  int64_t q_cap, kv_cap;   // list capacities for the smallest tile
  int32_t split;           // dK/dV workgroups per (key tile, KV head); > 1: partial planes at `part`
};

bool sizes_ok(int32_t batch, int32_t total_q, int32_t total_kv, int32_t hq, int32_t hkv, int32_t d) {
  return batch >= 0 && total_q >= 0 && total_kv >= 0 && hq >= 1 && hkv >= 1 && d >= 1;
}

// Workgroups that share a GQA group's query heads per (key tile, KV head) in
// dK/dV: 1, unless the group holds at least 8 query heads and the key tiles
// alone give fewer than 4096 workgroups (with few KV heads one workgroup
// would walk every query head of its group, and the longest one would set the
// kernel's time); then doubled, up to 4096 workgroups, while it divides the
// group and leaves every workgroup at least 2 of its heads (a workgroup per
// head writes the most partial planes for the least work).
int32_t dkdv_heads_split(int32_t batch, int32_t total_kv, int32_t hq, int32_t hkv) {
  const int32_t group = hq / hkv;
  if (group < 8) return 1;
  const int64_t wgs = (((int64_t)total_kv + kKVTile - 1) / kKVTile + batch) * hkv;
  int32_t split = 1;
  while (group % (2 * split) == 0 && group / (2 * split) >= 2 && wgs * split < 4096) split *= 2;
  return split;
}

// split: dK/dV workgroups per (key tile, KV head), >= 1 (1: no partial planes)
Layout layout(int32_t batch, int32_t total_q, int32_t total_kv, int32_t hq, int32_t hkv, int32_t d,
              int32_t split) {
  Layout L;
  L.q_cap = ((int64_t)total_q + kMinTile - 1) / kMinTile + batch;
  L.kv_cap = ((int64_t)total_kv + kMinTile - 1) / kMinTile + batch;
  size_t off = 0;
  L.hdr = off;
  off += round_up(kHdrWords * sizeof(int32_t));
  L.seq = off;
  off += round_up((size_t)batch * sizeof(SeqInfo));
  L.q_list = off;
  off += round_up((size_t)L.q_cap * sizeof(int2));
  L.kv_list = off;
  off += round_up((size_t)L.kv_cap * sizeof(int2));
  L.delta = off;
  off += round_up((size_t)total_q * (size_t)hq * sizeof(float));
  L.lse2 = off;
  off += round_up((size_t)total_q * (size_t)hq * sizeof(float));
  L.split = split;
  L.part = off;
  if (L.split > 1) off += round_up(2 * (size_t)L.split * (size_t)total_kv * (size_t)hkv * (size_t)d * sizeof(float));
  L.total = off;
  return L;
}

struct Common {
  Layout L;
  char* ws;
  int64_t q_tiles_max, kv_tiles_max;
};

// What varies between the entry points: the token layout (THD, with slots
// from cu_seqlens_*_padded, or a batched layout with fixed slots of slot_q /
// slot_kv tokens), the chunk positions of the causal rule, and whether the
// backward adds into its outputs.
struct CallOpts {
  int32_t layout = kLayoutThd;
  int32_t slot_q = 0, slot_kv = 0;
  const int32_t* q_pos0 = nullptr;
  const int32_t* kv_pos0 = nullptr;
  int32_t accumulate = 0;
  uint32_t drop_t = 0;        // dropout byte threshold round(256 p), 0 = none
  uint64_t seed = 0;
  uint32_t offset = 0;
  float out_scale = 1.f;      // forward output multiplier
  float dq_scale = 0.f;       // backward dQ / dK multipliers (0: the softmax scale)
  float dk_scale = 0.f;
  float delta_scale = 1.f;    // backward: Delta is used times this
  const void* q8 = nullptr;   // E4M3 q and k for the forward's 8-bit scores
  const void* k8 = nullptr;
  bool no_split = false;      // backward: never split a GQA group over dK/dV workgroups
  int32_t tsq(int32_t batch) const { return layout == kLayoutSbhd ? batch : 1; }
};
constexpr CallOpts kThd = {};

// the largest tile any kernel moves by one buffer-range DMA, in rows
constexpr int64_t kMaxDmaRows = 256;

// Checks shared by both entry points.  Nothing is launched before they pass.
attn_thd_status check_common(const void* q, const void* k, const void* v,
                             const int32_t* cu_q, const int32_t* cu_kv, int32_t batch,
                             int32_t total_q, int32_t total_kv, int32_t hq, int32_t hkv,
                             int32_t d, float scale, int32_t mask_type, int32_t dtype,
                             void* workspace, size_t workspace_bytes, const CallOpts& geo,
                             Common& c) {
  if (!sizes_ok(batch, total_q, total_kv, hq, hkv, d)) return ATTN_THD_EINVAL;
  if (hq % hkv != 0) return ATTN_THD_EINVAL;
  if (d % 8 != 0 || d > 256) return ATTN_THD_EUNSUPPORTED;
  if (dtype != ATTN_THD_BF16 && dtype != ATTN_THD_FP16) return ATTN_THD_EUNSUPPORTED;
  if (mask_type != ATTN_THD_MASK_PADDING && mask_type != ATTN_THD_MASK_PADDING_CAUSAL &&
      mask_type != ATTN_THD_MASK_PADDING_CAUSAL_BOTTOM_RIGHT)
    return ATTN_THD_EUNSUPPORTED;
  if (!(scale > 0.f) || !std::isfinite(scale)) return ATTN_THD_EINVAL;
  // THD needs the real boundaries; the batched layouts default to full slots
  if (geo.layout == kLayoutThd && (!cu_q || !cu_kv)) return ATTN_THD_EINVAL;
  // every DMA range (rows x token stride) must stay below 2 GiB
  const int64_t ts = geo.tsq(batch);
  if (kMaxDmaRows * ts * (int64_t)(hq > hkv ? hq : hkv) * d * 2 > INT32_MAX) return ATTN_THD_EINVAL;
  if ((total_q > 0 && !q) || (total_kv > 0 && (!k || !v))) return ATTN_THD_EINVAL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v)) return ATTN_THD_EINVAL;
  // grid sizes and element offsets must fit the kernels' integer types
  const int64_t q_tiles = ((int64_t)total_q + kQTile - 1) / kQTile + batch;
  const int64_t kv_tiles = ((int64_t)total_kv + dkdv_tile(d) - 1) / dkdv_tile(d) + batch;
  if (q_tiles * hq > INT32_MAX || kv_tiles * hkv > INT32_MAX) return ATTN_THD_EINVAL;
  if ((int64_t)total_q * hq > INT32_MAX || (int64_t)total_kv + 256 > INT32_MAX) return ATTN_THD_EINVAL;
  // a workspace below attn_thd_workspace_size (one sized for a problem with
  // more key tokens and so fewer partial planes, say) takes a smaller split,
  // down to none
  int32_t split = geo.no_split ? 1 : dkdv_heads_split(batch, total_kv, hq, hkv);
  while (split > 1 && layout(batch, total_q, total_kv, hq, hkv, d, split).total > workspace_bytes)
    split /= 2;
  c.L = layout(batch, total_q, total_kv, hq, hkv, d, split);
  if (!workspace || workspace_bytes < c.L.total) return ATTN_THD_EWORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0) return ATTN_THD_EWORKSPACE;
  c.ws = static_cast<char*>(workspace);
  c.q_tiles_max = q_tiles;
  c.kv_tiles_max = kv_tiles;
  return ATTN_THD_OK;
}

SchedParams sched_params(const Common& c, const int32_t* cu_q, const int32_t* cu_kv,
                         const int32_t* cu_qp, const int32_t* cu_kp, int32_t batch,
                         int32_t total_q, int32_t total_kv, int q_tile, int kv_tile,
                         int32_t mask_type, const CallOpts& geo) {
  SchedParams s = {};
  s.cu_q = cu_q;
  s.cu_kv = cu_kv;
  s.cu_qp = cu_qp;
  s.cu_kp = cu_kp;
  s.batch = batch;
  s.total_q = total_q;
  s.total_kv = total_kv;
  s.q_tile = q_tile;
  s.kv_tile = kv_tile;
  s.causal = mask_type == ATTN_THD_MASK_PADDING ? 0
             : (mask_type == ATTN_THD_MASK_PADDING_CAUSAL_BOTTOM_RIGHT ? 2 : 1);
  s.layout = geo.layout;
  s.slot_q = geo.slot_q;
  s.slot_kv = geo.slot_kv;
  s.q_pos0 = geo.q_pos0;
  s.kv_pos0 = geo.kv_pos0;
  s.hdr = reinterpret_cast<int32_t*>(c.ws + c.L.hdr);
  s.seq = reinterpret_cast<SeqInfo*>(c.ws + c.L.seq);
  s.q_list = reinterpret_cast<int2*>(c.ws + c.L.q_list);
  s.kv_list = reinterpret_cast<int2*>(c.ws + c.L.kv_list);
  return s;
}

AttnParams attn_params(const Common& c, int32_t hq, int32_t hkv, int32_t d, float scale,
                       int32_t mask_type, const CallOpts& geo, int32_t batch) {
  AttnParams a = {};
  a.hdr = reinterpret_cast<const int32_t*>(c.ws + c.L.hdr);
  a.seq = reinterpret_cast<const SeqInfo*>(c.ws + c.L.seq);
  a.delta = reinterpret_cast<float*>(c.ws + c.L.delta);
  a.lse2 = reinterpret_cast<float*>(c.ws + c.L.lse2);
  a.hq = hq;
  a.hkv = hkv;
  a.group = hq / hkv;
  a.d = d;
  a.scale = scale;
  a.scale_log2e = scale * kLog2e;
  (void)mask_type;   // the causal diagonal reaches the kernels in the sequence table
  a.tsq = geo.tsq(batch);
  a.tskv = geo.tsq(batch);
  a.accumulate = geo.accumulate;
  a.drop_t = geo.drop_t;
  a.seed_lo = (uint32_t)geo.seed;
  a.seed_hi = (uint32_t)(geo.seed >> 32);
  a.drop_c3 = geo.offset * (uint32_t)hq;
  a.drop_scale = 256.f / (float)(256u - geo.drop_t);
  a.out_scale = geo.out_scale;
  a.delta_scale = geo.delta_scale;
  a.q8 = geo.q8;
  a.k8 = geo.k8;
  a.kv_split = 1;
  a.kv_heads = a.group;
  return a;
}

ZeroParams zero_params(const Common& c, int32_t batch, int rows, int width, bool kv_side,
                       void* t0, void* t1, float* lse, int lse_heads, const CallOpts& geo) {
  ZeroParams z = {};
  z.hdr = reinterpret_cast<const int32_t*>(c.ws + c.L.hdr);
  z.seq = reinterpret_cast<const SeqInfo*>(c.ws + c.L.seq);
  z.batch = batch;
  z.rows = rows;
  z.width = width;
  z.kv_side = kv_side ? 1 : 0;
  z.lse_heads = lse_heads;
  z.layout = geo.layout;
  z.slot = kv_side ? geo.slot_kv : geo.slot_q;
  z.t0 = t0;
  z.t1 = t1;
  z.lse = lse;
  return z;
}

#define ATTN_TRY(expr)                                   \
  do {                                                   \
    if ((expr) != hipSuccess) return ATTN_THD_ELAUNCH;   \
  } while (0)

// Optional per-stage event marks (benchmark instrumentation); a NULL entry
// is a boundary the caller does not time.
struct Marks {
  void* const* ev;
  int n;
  hipStream_t s;
  hipError_t mark(int i) const {
    return (ev && i < n && ev[i]) ? hipEventRecord(static_cast<hipEvent_t>(ev[i]), s) : hipSuccess;
  }
};

constexpr int kFwdStages = 3;   // scheduler, forward, zero fill
constexpr int kBwdStages = 5;   // scheduler, dQ (+ Delta), dK/dV, zero fill (q rows), zero fill (kv rows)

attn_thd_status fwd_impl(const void* q, const void* k, const void* v, void* out, float* lse,
                         const int32_t* cu_q, const int32_t* cu_kv, const int32_t* cu_qp,
                         const int32_t* cu_kp, int32_t batch, int32_t total_q, int32_t total_kv,
                         int32_t hq, int32_t hkv, int32_t d, float scale, int32_t mask_type,
                         int32_t dtype, void* workspace, size_t workspace_bytes, void* stream,
                         void* const* events, int32_t n_events, const CallOpts& geo) {
  Common c;
  attn_thd_status st = check_common(q, k, v, cu_q, cu_kv, batch, total_q, total_kv, hq, hkv, d,
                                    scale, mask_type, dtype, workspace, workspace_bytes, geo, c);
  if (st != ATTN_THD_OK) return st;
  if (total_q > 0 && (!out || !lse)) return ATTN_THD_EINVAL;
  if (!aligned16(out) || (reinterpret_cast<uintptr_t>(lse) & 3u)) return ATTN_THD_EINVAL;
  if (events && n_events != kFwdStages + 1) return ATTN_THD_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Marks m{events, n_events, s};
  const bool causal = mask_type != ATTN_THD_MASK_PADDING;

  ATTN_TRY(m.mark(0));
  ATTN_TRY(launch_sched(sched_params(c, cu_q, cu_kv, cu_qp, cu_kp, batch, total_q, total_kv,
                                     kQTile, 0, mask_type, geo), s));
  AttnParams a = attn_params(c, hq, hkv, d, scale, mask_type, geo, batch);
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.lse_out = lse;
  a.list = reinterpret_cast<const int2*>(c.ws + c.L.q_list);
  ATTN_TRY(m.mark(1));
  ATTN_TRY(launch_fwd(a, dtype, causal, (int)c.q_tiles_max, s));
  ATTN_TRY(m.mark(2));
  ATTN_TRY(launch_zero_fill(zero_params(c, batch, total_q, hq * d, false, out, nullptr, lse, hq, geo), s));
  ATTN_TRY(m.mark(3));
  return ATTN_THD_OK;
}

// Host checks of the backward; nothing is launched before they pass.
static attn_thd_status bwd_check(const void* q, const void* k, const void* v, const void* out,
                                 const void* dout, const float* lse, void* dq, void* dk,
                                 void* dv, const int32_t* cu_q, const int32_t* cu_kv,
                                 int32_t batch, int32_t total_q, int32_t total_kv, int32_t hq,
                                 int32_t hkv, int32_t d, float scale, int32_t mask_type,
                                 int32_t dtype, void* workspace, size_t workspace_bytes,
                                 void* const* events, int32_t n_events, const CallOpts& geo,
                                 Common& c) {
  attn_thd_status st = check_common(q, k, v, cu_q, cu_kv, batch, total_q, total_kv, hq, hkv, d,
                                    scale, mask_type, dtype, workspace, workspace_bytes, geo, c);
  if (st != ATTN_THD_OK) return st;
  if (total_q > 0 && (!out || !dout || !lse || !dq)) return ATTN_THD_EINVAL;
  if (total_kv > 0 && (!dk || !dv)) return ATTN_THD_EINVAL;
  if (!aligned16(out) || !aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) ||
      (reinterpret_cast<uintptr_t>(lse) & 3u))
    return ATTN_THD_EINVAL;
  if (events && n_events != kBwdStages + 1) return ATTN_THD_EINVAL;
  return ATTN_THD_OK;
}

attn_thd_status bwd_impl(const void* q, const void* k, const void* v, const void* out,
                         const void* dout, const float* lse, void* dq, void* dk, void* dv,
                         const int32_t* cu_q, const int32_t* cu_kv, const int32_t* cu_qp,
                         const int32_t* cu_kp, int32_t batch, int32_t total_q, int32_t total_kv,
                         int32_t hq, int32_t hkv, int32_t d, float scale, int32_t mask_type,
                         int32_t dtype, void* workspace, size_t workspace_bytes, void* stream,
                         void* const* events, int32_t n_events, const CallOpts& geo) {
  Common c;
  attn_thd_status st = bwd_check(q, k, v, out, dout, lse, dq, dk, dv, cu_q, cu_kv, batch, total_q,
                                 total_kv, hq, hkv, d, scale, mask_type, dtype, workspace,
                                 workspace_bytes, events, n_events, geo, c);
  if (st != ATTN_THD_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Marks m{events, n_events, s};
  const bool causal = mask_type != ATTN_THD_MASK_PADDING;
  const int kv_tile = dkdv_tile(d);

  ATTN_TRY(m.mark(0));
  ATTN_TRY(launch_sched(sched_params(c, cu_q, cu_kv, cu_qp, cu_kp, batch, total_q, total_kv,
                                     kQTile, kv_tile, mask_type, geo), s));
  AttnParams a = attn_params(c, hq, hkv, d, scale, mask_type, geo, batch);
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = out;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.list = reinterpret_cast<const int2*>(c.ws + c.L.q_list);
  ATTN_TRY(m.mark(1));
  // dQ also forms Delta and LSE * log2(e) for every row it owns and writes
  // them to the workspace for dK/dV
  if (geo.dq_scale != 0.f) a.scale = geo.dq_scale;
  ATTN_TRY(launch_dq(a, dtype, causal, (int)c.q_tiles_max, s));
  a.list = reinterpret_cast<const int2*>(c.ws + c.L.kv_list);
  if (geo.dk_scale != 0.f) a.scale = geo.dk_scale;
  ATTN_TRY(m.mark(2));
  if (c.L.split > 1) {
    // the group's query heads over c.L.split workgroups, then their sum
    a.kv_split = c.L.split;
    a.kv_heads = a.group / c.L.split;
    a.part = reinterpret_cast<float*>(c.ws + c.L.part);
    a.part_plane = (int64_t)total_kv * hkv * d;
  }
  ATTN_TRY(launch_dkdv(a, dtype, causal, (int)c.kv_tiles_max, s));
  if (c.L.split > 1) ATTN_TRY(launch_dkdv_reduce(a, dtype, (int)c.kv_tiles_max, s));
  ATTN_TRY(m.mark(3));
  // an accumulated output keeps every row the call does not reach
  if (!(geo.accumulate & kAccDq))
    ATTN_TRY(launch_zero_fill(zero_params(c, batch, total_q, hq * d, false, dq, nullptr, nullptr, 0, geo), s));
  ATTN_TRY(m.mark(4));
  if (!(geo.accumulate & kAccDkDv))
    ATTN_TRY(launch_zero_fill(zero_params(c, batch, total_kv, hkv * d, true, dk, dv, nullptr, 0, geo), s));
  ATTN_TRY(m.mark(5));
  return ATTN_THD_OK;
}

}  // namespace

extern "C" {

size_t attn_thd_workspace_size(int32_t batch, int32_t total_q, int32_t total_kv, int32_t hq,
                               int32_t hkv, int32_t d) {
  if (!sizes_ok(batch, total_q, total_kv, hq, hkv, d)) return 0;
  return layout(batch, total_q, total_kv, hq, hkv, d, dkdv_heads_split(batch, total_kv, hq, hkv)).total;
}

attn_thd_status attn_fwd_thd(const void* q, const void* k, const void* v, void* out, float* lse,
                             const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
                             const int32_t* cu_seqlens_q_padded,
                             const int32_t* cu_seqlens_kv_padded, int32_t batch, int32_t total_q,
                             int32_t total_kv, int32_t max_seqlen_q, int32_t max_seqlen_kv,
                             int32_t hq, int32_t hkv, int32_t d, float scale, int32_t mask_type,
                             int32_t dtype, void* workspace, size_t workspace_bytes,
                             void* stream) {
  (void)max_seqlen_q;
  (void)max_seqlen_kv;
  return fwd_impl(q, k, v, out, lse, cu_seqlens_q, cu_seqlens_kv, cu_seqlens_q_padded,
                  cu_seqlens_kv_padded, batch, total_q, total_kv, hq, hkv, d, scale, mask_type,
                  dtype, workspace, workspace_bytes, stream, nullptr, 0, kThd);
}

attn_thd_status attn_fwd_thd_timed(const void* q, const void* k, const void* v, void* out,
                                   float* lse, const int32_t* cu_seqlens_q,
                                   const int32_t* cu_seqlens_kv,
                                   const int32_t* cu_seqlens_q_padded,
                                   const int32_t* cu_seqlens_kv_padded, int32_t batch,
                                   int32_t total_q, int32_t total_kv, int32_t max_seqlen_q,
                                   int32_t max_seqlen_kv, int32_t hq, int32_t hkv, int32_t d,
                                   float scale, int32_t mask_type, int32_t dtype, void* workspace,
                                   size_t workspace_bytes, void* stream, void* const* events,
                                   int32_t n_events) {
  (void)max_seqlen_q;
  (void)max_seqlen_kv;
  if (!events) return ATTN_THD_EINVAL;
  return fwd_impl(q, k, v, out, lse, cu_seqlens_q, cu_seqlens_kv, cu_seqlens_q_padded,
                  cu_seqlens_kv_padded, batch, total_q, total_kv, hq, hkv, d, scale, mask_type,
                  dtype, workspace, workspace_bytes, stream, events, n_events, kThd);
}

attn_thd_status attn_bwd_thd(const void* q, const void* k, const void* v, const void* out,
                             const void* dout, const float* lse, void* dq, void* dk, void* dv,
                             const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
                             const int32_t* cu_seqlens_q_padded,
                             const int32_t* cu_seqlens_kv_padded, int32_t batch, int32_t total_q,
                             int32_t total_kv, int32_t max_seqlen_q, int32_t max_seqlen_kv,
                             int32_t hq, int32_t hkv, int32_t d, float scale, int32_t mask_type,
                             int32_t dtype, void* workspace, size_t workspace_bytes,
                             void* stream) {
  (void)max_seqlen_q;
  (void)max_seqlen_kv;
  return bwd_impl(q, k, v, out, dout, lse, dq, dk, dv, cu_seqlens_q, cu_seqlens_kv,
                  cu_seqlens_q_padded, cu_seqlens_kv_padded, batch, total_q, total_kv, hq, hkv, d,
                  scale, mask_type, dtype, workspace, workspace_bytes, stream, nullptr, 0, kThd);
}

attn_thd_status attn_bwd_thd_timed(const void* q, const void* k, const void* v, const void* out,
                                   const void* dout, const float* lse, void* dq, void* dk,
                                   void* dv, const int32_t* cu_seqlens_q,
                                   const int32_t* cu_seqlens_kv,
                                   const int32_t* cu_seqlens_q_padded,
                                   const int32_t* cu_seqlens_kv_padded, int32_t batch,
                                   int32_t total_q, int32_t total_kv, int32_t max_seqlen_q,
                                   int32_t max_seqlen_kv, int32_t hq, int32_t hkv, int32_t d,
                                   float scale, int32_t mask_type, int32_t dtype, void* workspace,
                                   size_t workspace_bytes, void* stream, void* const* events,
                                   int32_t n_events) {
  (void)max_seqlen_q;
  (void)max_seqlen_kv;
  if (!events) return ATTN_THD_EINVAL;
  return bwd_impl(q, k, v, out, dout, lse, dq, dk, dv, cu_seqlens_q, cu_seqlens_kv,
                  cu_seqlens_q_padded, cu_seqlens_kv_padded, batch, total_q, total_kv, hq, hkv, d,
                  scale, mask_type, dtype, workspace, workspace_bytes, stream, events, n_events, kThd);
}

// Batched layouts: geometry checks, then the THD path with fixed slots.
static attn_thd_status batched_geom(int32_t layout, int32_t batch, int32_t seqlen_q,
                                    int32_t seqlen_kv, CallOpts& geo, int32_t& total_q,
                                    int32_t& total_kv) {
  if (layout != ATTN_THD_LAYOUT_BSHD && layout != ATTN_THD_LAYOUT_SBHD) return ATTN_THD_EUNSUPPORTED;
  if (batch < 0 || seqlen_q < 0 || seqlen_kv < 0) return ATTN_THD_EINVAL;
  const int64_t tq = (int64_t)batch * seqlen_q, tk = (int64_t)batch * seqlen_kv;
  if (tq > INT32_MAX || tk > INT32_MAX) return ATTN_THD_EINVAL;
  geo.layout = layout == ATTN_THD_LAYOUT_BSHD ? kLayoutBshd : kLayoutSbhd;
  geo.slot_q = seqlen_q;
  geo.slot_kv = seqlen_kv;
  total_q = (int32_t)tq;
  total_kv = (int32_t)tk;
  return ATTN_THD_OK;
}

static attn_thd_status fwd_batched(const void* q, const void* k, const void* v, void* out,
                                   float* lse, const int32_t* cu_q, const int32_t* cu_kv,
                                   int32_t layout, int32_t batch, int32_t seqlen_q,
                                   int32_t seqlen_kv, int32_t hq, int32_t hkv, int32_t d,
                                   float scale, int32_t mask_type, int32_t dtype, void* workspace,
                                   size_t workspace_bytes, void* stream, void* const* events,
                                   int32_t n_events) {
  CallOpts geo = kThd;   // batched_geom sets the layout fields only
  int32_t total_q, total_kv;
  attn_thd_status st = batched_geom(layout, batch, seqlen_q, seqlen_kv, geo, total_q, total_kv);
  if (st != ATTN_THD_OK) return st;
  return fwd_impl(q, k, v, out, lse, cu_q, cu_kv, nullptr, nullptr, batch, total_q, total_kv, hq,
                  hkv, d, scale, mask_type, dtype, workspace, workspace_bytes, stream, events,
                  n_events, geo);
}

static attn_thd_status bwd_batched(const void* q, const void* k, const void* v, const void* out,
                                   const void* dout, const float* lse, void* dq, void* dk,
                                   void* dv, const int32_t* cu_q, const int32_t* cu_kv,
                                   int32_t layout, int32_t batch, int32_t seqlen_q,
                                   int32_t seqlen_kv, int32_t hq, int32_t hkv, int32_t d,
                                   float scale, int32_t mask_type, int32_t dtype, void* workspace,
                                   size_t workspace_bytes, void* stream, void* const* events,
                                   int32_t n_events) {
  CallOpts geo = kThd;   // batched_geom sets the layout fields only
  int32_t total_q, total_kv;
  attn_thd_status st = batched_geom(layout, batch, seqlen_q, seqlen_kv, geo, total_q, total_kv);
  if (st != ATTN_THD_OK) return st;
  return bwd_impl(q, k, v, out, dout, lse, dq, dk, dv, cu_q, cu_kv, nullptr, nullptr, batch,
                  total_q, total_kv, hq, hkv, d, scale, mask_type, dtype, workspace,
                  workspace_bytes, stream, events, n_events, geo);
}

attn_thd_status attn_fwd_batched(const void* q, const void* k, const void* v, void* out,
                                 float* lse, const int32_t* cu_seqlens_q,
                                 const int32_t* cu_seqlens_kv, int32_t layout, int32_t batch,
                                 int32_t seqlen_q, int32_t seqlen_kv, int32_t hq, int32_t hkv,
                                 int32_t d, float scale, int32_t mask_type, int32_t dtype,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  return fwd_batched(q, k, v, out, lse, cu_seqlens_q, cu_seqlens_kv, layout, batch, seqlen_q,
                     seqlen_kv, hq, hkv, d, scale, mask_type, dtype, workspace, workspace_bytes,
                     stream, nullptr, 0);
}

attn_thd_status attn_bwd_batched(const void* q, const void* k, const void* v, const void* out,
                                 const void* dout, const float* lse, void* dq, void* dk, void* dv,
                                 const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
                                 int32_t layout, int32_t batch, int32_t seqlen_q,
                                 int32_t seqlen_kv, int32_t hq, int32_t hkv, int32_t d,
                                 float scale, int32_t mask_type, int32_t dtype, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  return bwd_batched(q, k, v, out, dout, lse, dq, dk, dv, cu_seqlens_q, cu_seqlens_kv, layout,
                     batch, seqlen_q, seqlen_kv, hq, hkv, d, scale, mask_type, dtype, workspace,
                     workspace_bytes, stream, nullptr, 0);
}

attn_thd_status attn_fwd_batched_timed(const void* q, const void* k, const void* v, void* out,
                                       float* lse, const int32_t* cu_seqlens_q,
                                       const int32_t* cu_seqlens_kv, int32_t layout,
                                       int32_t batch, int32_t seqlen_q, int32_t seqlen_kv,
                                       int32_t hq, int32_t hkv, int32_t d, float scale,
                                       int32_t mask_type, int32_t dtype, void* workspace,
                                       size_t workspace_bytes, void* stream, void* const* events,
                                       int32_t n_events) {
  if (!events) return ATTN_THD_EINVAL;
  return fwd_batched(q, k, v, out, lse, cu_seqlens_q, cu_seqlens_kv, layout, batch, seqlen_q,
                     seqlen_kv, hq, hkv, d, scale, mask_type, dtype, workspace, workspace_bytes,
                     stream, events, n_events);
}

attn_thd_status attn_bwd_batched_timed(const void* q, const void* k, const void* v,
                                       const void* out, const void* dout, const float* lse,
                                       void* dq, void* dk, void* dv, const int32_t* cu_seqlens_q,
                                       const int32_t* cu_seqlens_kv, int32_t layout,
                                       int32_t batch, int32_t seqlen_q, int32_t seqlen_kv,
                                       int32_t hq, int32_t hkv, int32_t d, float scale,
                                       int32_t mask_type, int32_t dtype, void* workspace,
                                       size_t workspace_bytes, void* stream, void* const* events,
                                       int32_t n_events) {
  if (!events) return ATTN_THD_EINVAL;
  return bwd_batched(q, k, v, out, dout, lse, dq, dk, dv, cu_seqlens_q, cu_seqlens_kv, layout,
                     batch, seqlen_q, seqlen_kv, hq, hkv, d, scale, mask_type, dtype, workspace,
                     workspace_bytes, stream, events, n_events);
}

// ----------------------------------------------------------------- dropout
// Byte threshold of a dropout probability: round(256 p) for p in [0, 255.5/256).
static bool dropout_threshold(float p, uint32_t& t) {
  if (!(p >= 0.f) || !(p < 255.5f / 256.f)) return false;
  t = (uint32_t)std::floor(256.0 * (double)p + 0.5);
  return true;
}

attn_thd_status attn_fwd_thd_dropout(const void* q, const void* k, const void* v, void* out,
                                     float* lse, const int32_t* cu_seqlens_q,
                                     const int32_t* cu_seqlens_kv,
                                     const int32_t* cu_seqlens_q_padded,
                                     const int32_t* cu_seqlens_kv_padded, int32_t batch,
                                     int32_t total_q, int32_t total_kv, int32_t hq, int32_t hkv,
                                     int32_t d, float scale, int32_t mask_type, float dropout_p,
                                     uint64_t seed, uint32_t offset, int32_t dtype,
                                     void* workspace, size_t workspace_bytes, void* stream,
                                     void* const* events, int32_t n_events) {
  CallOpts o = kThd;
  if (!dropout_threshold(dropout_p, o.drop_t)) return ATTN_THD_EINVAL;
  o.seed = seed;
  o.offset = offset;
  return fwd_impl(q, k, v, out, lse, cu_seqlens_q, cu_seqlens_kv, cu_seqlens_q_padded,
                  cu_seqlens_kv_padded, batch, total_q, total_kv, hq, hkv, d, scale, mask_type,
                  dtype, workspace, workspace_bytes, stream, events, n_events, o);
}

attn_thd_status attn_bwd_thd_dropout(const void* q, const void* k, const void* v, const void* out,
                                     const void* dout, const float* lse, void* dq, void* dk,
                                     void* dv, const int32_t* cu_seqlens_q,
                                     const int32_t* cu_seqlens_kv,
                                     const int32_t* cu_seqlens_q_padded,
                                     const int32_t* cu_seqlens_kv_padded, int32_t batch,
                                     int32_t total_q, int32_t total_kv, int32_t hq, int32_t hkv,
                                     int32_t d, float scale, int32_t mask_type, float dropout_p,
                                     uint64_t seed, uint32_t offset, int32_t dtype,
                                     void* workspace, size_t workspace_bytes, void* stream,
                                     void* const* events, int32_t n_events) {
  CallOpts o = kThd;
  if (!dropout_threshold(dropout_p, o.drop_t)) return ATTN_THD_EINVAL;
  o.seed = seed;
  o.offset = offset;
  return bwd_impl(q, k, v, out, dout, lse, dq, dk, dv, cu_seqlens_q, cu_seqlens_kv,
                  cu_seqlens_q_padded, cu_seqlens_kv_padded, batch, total_q, total_kv, hq, hkv, d,
                  scale, mask_type, dtype, workspace, workspace_bytes, stream, events, n_events, o);
}

// ----------------------------------------------------------------- FP8 inputs
// Workspace of the FP8 forward: the plain layout, then 16-bit copies of q, k
// and v (each 256-byte aligned).
struct Fp8Layout {
  size_t base, q, k, v, total;
};
static Fp8Layout fp8_layout(int32_t batch, int32_t total_q, int32_t total_kv, int32_t hq,
                            int32_t hkv, int32_t d) {
  Fp8Layout f;
  f.base = layout(batch, total_q, total_kv, hq, hkv, d, dkdv_heads_split(batch, total_kv, hq, hkv)).total;
  f.q = f.base;
  f.k = f.q + round_up((size_t)total_q * hq * d * 2);
  f.v = f.k + round_up((size_t)total_kv * hkv * d * 2);
  f.total = f.v + round_up((size_t)total_kv * hkv * d * 2);
  return f;
}

size_t attn_thd_fp8_workspace_size(int32_t batch, int32_t total_q, int32_t total_kv, int32_t hq,
                                   int32_t hkv, int32_t d) {
  if (!sizes_ok(batch, total_q, total_kv, hq, hkv, d)) return 0;
  return fp8_layout(batch, total_q, total_kv, hq, hkv, d).total;
}

attn_thd_status attn_fwd_thd_fp8(const void* q8, const void* k8, const void* v8, float descale_q,
                                 float descale_k, float descale_v, void* out, float* lse,
                                 const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
                                 const int32_t* cu_seqlens_q_padded,
                                 const int32_t* cu_seqlens_kv_padded, int32_t batch,
                                 int32_t total_q, int32_t total_kv, int32_t hq, int32_t hkv,
                                 int32_t d, float scale, int32_t mask_type, int32_t out_dtype,
                                 void* workspace, size_t workspace_bytes, void* stream,
                                 void* const* events, int32_t n_events) {
  if (!sizes_ok(batch, total_q, total_kv, hq, hkv, d)) return ATTN_THD_EINVAL;
  if (events && n_events != kFwdStages + 2) return ATTN_THD_EINVAL;
  for (float s : {descale_q, descale_k, descale_v})
    if (!(s > 0.f) || !std::isfinite(s)) return ATTN_THD_EINVAL;
  if (!(scale > 0.f) || !std::isfinite(scale) || !std::isfinite(scale * descale_q * descale_k) ||
      !(scale * descale_q * descale_k > 0.f))
    return ATTN_THD_EINVAL;
  if ((total_q > 0 && !q8) || (total_kv > 0 && (!k8 || !v8))) return ATTN_THD_EINVAL;
  // 8 codes per load: rows of d (a multiple of 8) bytes need 8-byte alignment
  auto al8 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; };
  if (!al8(q8) || !al8(k8) || !al8(v8)) return ATTN_THD_EINVAL;
  if (d % 8 != 0 || d > 256) return ATTN_THD_EUNSUPPORTED;
  if (out_dtype != ATTN_THD_BF16 && out_dtype != ATTN_THD_FP16) return ATTN_THD_EUNSUPPORTED;
  const Fp8Layout f = fp8_layout(batch, total_q, total_kv, hq, hkv, d);
  char* ws = static_cast<char*>(workspace);
  void* q16 = ws + f.q;
  void* k16 = ws + f.k;
  void* v16 = ws + f.v;
  // head dims 48..256 (multiples of 16) with 16-byte aligned codes take the
  // scores on the 8-bit products straight from q8 / k8 (64-code chunks, the
  // last one zero-padded past d); other shapes decode q and k too and run the
  // 16-bit forward
  const bool s8 = d % 16 == 0 && d > 32 && d <= 256 && aligned16(q8) && aligned16(k8);
  // the forward's own checks first (in its order), so that nothing is
  // launched on bad arguments; then room for the decoded copies
  Common c;
  attn_thd_status st = check_common(s8 ? q8 : q16, s8 ? k8 : k16, v16, cu_seqlens_q, cu_seqlens_kv,
                                    batch, total_q, total_kv, hq, hkv, d,
                                    scale * descale_q * descale_k, mask_type, out_dtype, workspace,
                                    f.base, kThd, c);
  if (st != ATTN_THD_OK) return st;
  if (workspace_bytes < f.total) return ATTN_THD_EWORKSPACE;
  if (total_q > 0 && (!out || !lse)) return ATTN_THD_EINVAL;
  if (!aligned16(out) || (reinterpret_cast<uintptr_t>(lse) & 3u)) return ATTN_THD_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Marks m{events, n_events, s};
  ATTN_TRY(m.mark(0));
  if (!s8) {
    ATTN_TRY(launch_decode_e4m3(q8, q16, (int64_t)total_q * hq * d, out_dtype, s));
    ATTN_TRY(launch_decode_e4m3(k8, k16, (int64_t)total_kv * hkv * d, out_dtype, s));
  }
  ATTN_TRY(launch_decode_e4m3(v8, v16, (int64_t)total_kv * hkv * d, out_dtype, s));
  CallOpts o = kThd;
  o.out_scale = descale_v;
  if (s8) {
    o.q8 = q8;
    o.k8 = k8;
  }
  // the forward marks events[1..4]
  return fwd_impl(q16, k16, v16, out, lse, cu_seqlens_q, cu_seqlens_kv, cu_seqlens_q_padded,
                  cu_seqlens_kv_padded, batch, total_q, total_kv, hq, hkv, d,
                  scale * descale_q * descale_k, mask_type, out_dtype, workspace, f.base, stream,
                  events ? events + 1 : nullptr, events ? n_events - 1 : 0, o);
}

attn_thd_status attn_bwd_thd_fp8(const void* q8, const void* k8, const void* v8, float descale_q,
                                 float descale_k, float descale_v, const void* out,
                                 const void* dout, const float* lse, void* dq, void* dk,
                                 void* dv, const int32_t* cu_seqlens_q,
                                 const int32_t* cu_seqlens_kv,
                                 const int32_t* cu_seqlens_q_padded,
                                 const int32_t* cu_seqlens_kv_padded, int32_t batch,
                                 int32_t total_q, int32_t total_kv, int32_t hq, int32_t hkv,
                                 int32_t d, float scale, int32_t mask_type, int32_t dtype,
                                 void* workspace, size_t workspace_bytes, void* stream,
                                 void* const* events, int32_t n_events) {
  if (!sizes_ok(batch, total_q, total_kv, hq, hkv, d)) return ATTN_THD_EINVAL;
  if (events && n_events != kBwdStages + 2) return ATTN_THD_EINVAL;
  for (float s : {descale_q, descale_k, descale_v})
    if (!(s > 0.f) || !std::isfinite(s)) return ATTN_THD_EINVAL;
  // the three factors the kernels take: the score scale, and the dQ / dK
  // multipliers of dS' = dS / descale_v
  const float s_qk = scale * descale_q * descale_k;
  const float f_dq = scale * descale_k * descale_v, f_dk = scale * descale_q * descale_v;
  for (float f : {s_qk, f_dq, f_dk, 1.f / descale_v})
    if (!(f > 0.f) || !std::isfinite(f)) return ATTN_THD_EINVAL;
  if (!(scale > 0.f) || !std::isfinite(scale)) return ATTN_THD_EINVAL;
  if ((total_q > 0 && !q8) || (total_kv > 0 && (!k8 || !v8))) return ATTN_THD_EINVAL;
  auto al8 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; };
  if (!al8(q8) || !al8(k8) || !al8(v8)) return ATTN_THD_EINVAL;
  if (d % 8 != 0 || d > 256) return ATTN_THD_EUNSUPPORTED;
  if (dtype != ATTN_THD_BF16 && dtype != ATTN_THD_FP16) return ATTN_THD_EUNSUPPORTED;
  const Fp8Layout f = fp8_layout(batch, total_q, total_kv, hq, hkv, d);
  char* ws = static_cast<char*>(workspace);
  void* q16 = ws + f.q;
  void* k16 = ws + f.k;
  void* v16 = ws + f.v;
  CallOpts o = kThd;
  o.dq_scale = f_dq;
  o.dk_scale = f_dk;
  o.delta_scale = 1.f / descale_v;
  // the backward's own checks first, so that nothing is launched on bad
  // arguments; then room for the decoded copies
  Common c;
  attn_thd_status st = bwd_check(q16, k16, v16, out, dout, lse, dq, dk, dv, cu_seqlens_q,
                                 cu_seqlens_kv, batch, total_q, total_kv, hq, hkv, d, s_qk,
                                 mask_type, dtype, workspace, f.base,
                                 events ? events + 1 : nullptr, events ? n_events - 1 : 0, o, c);
  if (st != ATTN_THD_OK) return st;
  if (workspace_bytes < f.total) return ATTN_THD_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Marks m{events, n_events, s};
  ATTN_TRY(m.mark(0));
  // the codes themselves (exact in both 16-bit types); the descales enter
  // through s_qk, f_dq, f_dk and the Delta factor
  ATTN_TRY(launch_decode_e4m3(q8, q16, (int64_t)total_q * hq * d, dtype, s));
  ATTN_TRY(launch_decode_e4m3(k8, k16, (int64_t)total_kv * hkv * d, dtype, s));
  ATTN_TRY(launch_decode_e4m3(v8, v16, (int64_t)total_kv * hkv * d, dtype, s));
  // the backward marks events[1..]
  return bwd_impl(q16, k16, v16, out, dout, lse, dq, dk, dv, cu_seqlens_q, cu_seqlens_kv,
                  cu_seqlens_q_padded, cu_seqlens_kv_padded, batch, total_q, total_kv, hq, hkv, d,
                  s_qk, mask_type, dtype, workspace, f.base, stream,
                  events ? events + 1 : nullptr, events ? n_events - 1 : 0, o);
}

// ----------------------------------------------------------------- chunked form
attn_thd_status attn_fwd_thd_chunk(const void* q, const void* k, const void* v, void* out,
                                   float* lse, const int32_t* cu_seqlens_q,
                                   const int32_t* cu_seqlens_kv,
                                   const int32_t* cu_seqlens_q_padded,
                                   const int32_t* cu_seqlens_kv_padded, const int32_t* q_pos0,
                                   const int32_t* kv_pos0, int32_t batch, int32_t total_q,
                                   int32_t total_kv, int32_t hq, int32_t hkv, int32_t d,
                                   float scale, int32_t mask_type, int32_t dtype, void* workspace,
                                   size_t workspace_bytes, void* stream, void* const* events,
                                   int32_t n_events) {
  if ((q_pos0 || kv_pos0) && mask_type != ATTN_THD_MASK_PADDING_CAUSAL) return ATTN_THD_EINVAL;
  CallOpts o = kThd;
  o.q_pos0 = q_pos0;
  o.kv_pos0 = kv_pos0;
  return fwd_impl(q, k, v, out, lse, cu_seqlens_q, cu_seqlens_kv, cu_seqlens_q_padded,
                  cu_seqlens_kv_padded, batch, total_q, total_kv, hq, hkv, d, scale, mask_type,
                  dtype, workspace, workspace_bytes, stream, events, n_events, o);
}

attn_thd_status attn_bwd_thd_chunk(const void* q, const void* k, const void* v, const void* out,
                                   const void* dout, const float* lse, void* dq, void* dk,
                                   void* dv, const int32_t* cu_seqlens_q,
                                   const int32_t* cu_seqlens_kv,
                                   const int32_t* cu_seqlens_q_padded,
                                   const int32_t* cu_seqlens_kv_padded, const int32_t* q_pos0,
                                   const int32_t* kv_pos0, int32_t batch, int32_t total_q,
                                   int32_t total_kv, int32_t hq, int32_t hkv, int32_t d,
                                   float scale, int32_t mask_type, int32_t accumulate,
                                   int32_t dtype, void* workspace, size_t workspace_bytes,
                                   void* stream, void* const* events, int32_t n_events) {
  if ((q_pos0 || kv_pos0) && mask_type != ATTN_THD_MASK_PADDING_CAUSAL) return ATTN_THD_EINVAL;
  if (accumulate & ~(ATTN_THD_ACC_DQ | ATTN_THD_ACC_DKDV)) return ATTN_THD_EINVAL;
  CallOpts o = kThd;
  o.q_pos0 = q_pos0;
  o.kv_pos0 = kv_pos0;
  o.accumulate = accumulate;
  return bwd_impl(q, k, v, out, dout, lse, dq, dk, dv, cu_seqlens_q, cu_seqlens_kv,
                  cu_seqlens_q_padded, cu_seqlens_kv_padded, batch, total_q, total_kv, hq, hkv, d,
                  scale, mask_type, dtype, workspace, workspace_bytes, stream, events, n_events, o);
}

attn_thd_status attn_merge_thd(void* out, float* lse, const void* out_part,
                               const float* lse_part, int32_t total_q, int32_t hq, int32_t d,
                               int32_t dtype, void* stream) {
  if (total_q < 0 || hq < 1 || d < 1) return ATTN_THD_EINVAL;
  if (d % 8 != 0 || d > 256) return ATTN_THD_EUNSUPPORTED;
  if (dtype != ATTN_THD_BF16 && dtype != ATTN_THD_FP16) return ATTN_THD_EUNSUPPORTED;
  if ((int64_t)total_q * hq > INT32_MAX) return ATTN_THD_EINVAL;
  if (total_q > 0 && (!out || !lse || !out_part || !lse_part)) return ATTN_THD_EINVAL;
  if (!aligned16(out) || !aligned16(out_part) || (reinterpret_cast<uintptr_t>(lse) & 3u) ||
      (reinterpret_cast<uintptr_t>(lse_part) & 3u))
    return ATTN_THD_EINVAL;
  if (launch_merge(out, lse, out_part, lse_part, (int64_t)total_q * hq, d, dtype,
                   static_cast<hipStream_t>(stream)) != hipSuccess)
    return ATTN_THD_ELAUNCH;
  return ATTN_THD_OK;
}

}  // extern "C"

// ----------------------------------------------------------------- no-allocation backward
// Scratch of attn_bwd_thd_noalloc: each GPU the library runs on holds its own
// copy of this array.  In host code the name is only a stand-in for the
// symbol; the device address of the current GPU's copy comes from
// hipGetSymbolAddress and is the only form passed to kernels.
static __device__ __align__(256) unsigned char scratch[ATTN_THD_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];   // device address of `scratch`, per device

// The current device's copy of `scratch`, looked up on the first call there.
// Two threads racing on a first call both store the same address.
attn_thd_status scratch_for(void* stream, void** ptr) {
  int dev = -1, sdev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ATTN_THD_ELAUNCH;
  if (stream) {
    if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev) != hipSuccess) return ATTN_THD_EINVAL;
    if (sdev != dev) return ATTN_THD_EINVAL;
  }
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return ATTN_THD_ELAUNCH;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return ATTN_THD_OK;
}

}  // namespace

extern "C" {

attn_thd_status attn_bwd_thd_noalloc(const void* q, const void* k, const void* v, const void* out,
                                     const void* dout, const float* lse, void* dq, void* dk,
                                     void* dv, const int32_t* cu_seqlens_q,
                                     const int32_t* cu_seqlens_kv,
                                     const int32_t* cu_seqlens_q_padded,
                                     const int32_t* cu_seqlens_kv_padded, int32_t batch,
                                     int32_t total_q, int32_t total_kv, int32_t max_seqlen_q,
                                     int32_t max_seqlen_kv, int32_t hq, int32_t hkv, int32_t d,
                                     float scale, int32_t mask_type, int32_t dtype, void* stream) {
  (void)max_seqlen_q;
  (void)max_seqlen_kv;
  if (!sizes_ok(batch, total_q, total_kv, hq, hkv, d)) return ATTN_THD_EINVAL;
  // the unsplit dK/dV: the scratch holds no partial planes
  if (layout(batch, total_q, total_kv, hq, hkv, d, 1).total > ATTN_THD_NOALLOC_SCRATCH_BYTES)
    return ATTN_THD_ESCRATCH;
  void* ws = nullptr;
  const attn_thd_status st = scratch_for(stream, &ws);
  if (st != ATTN_THD_OK) return st;
  CallOpts o = kThd;
  o.no_split = true;
  return bwd_impl(q, k, v, out, dout, lse, dq, dk, dv, cu_seqlens_q, cu_seqlens_kv,
                  cu_seqlens_q_padded, cu_seqlens_kv_padded, batch, total_q, total_kv, hq, hkv, d,
                  scale, mask_type, dtype, ws, ATTN_THD_NOALLOC_SCRATCH_BYTES, stream, nullptr, 0, o);
}

const char* attn_thd_status_string(int32_t status) {
  switch (status) {
    case ATTN_THD_OK: return "ok";
    case ATTN_THD_EINVAL: return "invalid argument";
    case ATTN_THD_EUNSUPPORTED: return "unsupported head dim, dtype or mask";
    case ATTN_THD_EWORKSPACE: return "workspace missing, too small or misaligned";
    case ATTN_THD_ELAUNCH: return "kernel launch failed";
    case ATTN_THD_ESCRATCH: return "problem exceeds the static scratch of the no-allocation backward";
    default: return "unknown status";
  }
}

attn_thd_status attn_thd_read_device_status(const void* workspace, void* stream, int32_t* status_out) {
  if (!workspace || !status_out) return ATTN_THD_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (hipStreamSynchronize(s) != hipSuccess) return ATTN_THD_ELAUNCH;
  int32_t v = 0;
  if (hipMemcpy(&v, workspace, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess) return ATTN_THD_ELAUNCH;
  *status_out = v;
  return ATTN_THD_OK;
}

}  // extern "C"
