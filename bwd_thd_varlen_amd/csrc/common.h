// Shared device definitions for the gfx950 THD attention kernels.
//
// MFMA layout used throughout (v_mfma_f32_32x32x16_{bf16,f16}, wave64):
//   * A operand (32 rows x 16 k): lane l supplies row (l & 31) and 8 k-values;
//     B operand (16 k x 32 cols): lane l supplies column (l & 31) and 8 k-values.
//     The hardware pairs A-slot s of lane half (l >> 5) with B-slot s of the
//     same half, so any assignment of k indices to (half, slot) works as long
//     as A and B use the same one.  Here slot s of half hh holds
//     k = 8*hh + s when both operands come from memory, and the "P-order"
//     k = 8*(s/4) + 4*hh + (s%4) when one operand is an accumulator tile
//     reused as an input (see below).
//   * C/D (32 x 32 fp32): lane l holds column (l & 31); register r holds row
//     8*(r/4) + 4*(l >> 5) + (r%4).
// An accumulator tile C read column-by-lane therefore already has, for a
// 16-row chunk u, the rows 16u + 8*(s/4) + 4*hh + (s%4) in registers
// 8*(u%2) + s: exactly a B (or A) operand in P-order.  A second operand that
// must match is stored in LDS transposed with the matching permutation of its
// contraction index inside each 16-block (perm16), so one 16-byte LDS read
// yields it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kBF16 = 0;
constexpr int kFP16 = 1;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Tile geometry shared by host and device.
constexpr int kQTile = 128;      // query rows per forward / dQ work item (4 waves x 32)
constexpr int kKVStep = 64;      // keys per inner step of the forward / dQ kernels
constexpr int kMinTile = 64;     // smallest tile any list uses (sizes the lists)
constexpr int kSchedKeys = 2048; // distinct work keys of the longest-first ordering

// Workspace header (int32 words at the start of the workspace).
constexpr int kHdrStatus = 0;
constexpr int kHdrNQTiles = 1;
constexpr int kHdrNKVTiles = 2;
constexpr int kHdrWords = 64;    // 256 bytes

// Per-sequence record written by the scheduler.
struct SeqInfo {
  int32_t oq, lq, ok, lk;        // padded offsets and real lengths
};

template <int DT> struct Mfma;

template <> struct Mfma<kBF16> {
  static __device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  // two fp32 -> two bf16 (round to nearest even), low half = a
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
  }
};

template <> struct Mfma<kFP16> {
  static __device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, f16x2));
  }
};

// Eight consecutive accumulator registers [8*half8, 8*half8+8) of a C tile,
// rounded to the storage dtype and packed as an MFMA operand (P-order).
template <int DT>
__device__ __forceinline__ u32x4 pack_operand(const f32x16& c, int half8) {
  const int o = 8 * half8;
  u32x4 r;
  r[0] = Mfma<DT>::pack2(c[o + 0], c[o + 1]);
  r[1] = Mfma<DT>::pack2(c[o + 2], c[o + 3]);
  r[2] = Mfma<DT>::pack2(c[o + 4], c[o + 5]);
  r[3] = Mfma<DT>::pack2(c[o + 6], c[o + 7]);
  return r;
}

// Position of contraction index j inside its 16-block when stored for a
// P-order operand: swaps bits 2 and 3 so that lane half hh finds its eight
// values j = 8a + 4hh + p (a in {0,1}, p in 0..3) at 8hh + 4a + p.
__device__ __forceinline__ int perm16(int j) {
  return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

__device__ __forceinline__ u32x4 ldg16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Maps a linear workgroup id onto (work item, head) so that the heads an
// XCD receives are contiguous (they share K/V tiles in that XCD's L2).
// Workgroups are dispatched round-robin over the 8 XCDs by id.  Falls back
// to the plain order when `heads` is not a multiple of 8.
__device__ __forceinline__ void xcd_split(int L, int heads, int& item, int& head) {
  if ((heads & 7) == 0) {
    const int per = heads >> 3;
    const int x = L & 7, j = L >> 3;
    item = j / per;
    head = x * per + (j - (j / per) * per);
  } else {
    item = L / heads;
    head = L - item * heads;
  }
}

// ----------------------------------------------------------------- kernel params
struct SchedParams {
  const int32_t* cu_q;
  const int32_t* cu_kv;
  const int32_t* cu_qp;
  const int32_t* cu_kp;
  int32_t batch, total_q, total_kv;
  int32_t q_tile, kv_tile;       // 0 = do not build that list
  int32_t causal;
  int32_t* hdr;
  SeqInfo* seq;
  int2* q_list;
  int2* kv_list;
};

struct ZeroParams {
  const int32_t* hdr;
  const SeqInfo* seq;
  int32_t batch, rows, width;    // width = heads * d elements per row
  int32_t kv_side;               // 0: query rows (out/dq, lse); 1: key rows (dk, dv)
  int32_t lse_heads;             // heads of lse (0 = no lse to write)
  void* t0;
  void* t1;
  float* lse;
};

struct AttnParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* out;       // forward output
  float* lse_out;  // forward lse
  void* dq;
  void* dk;
  void* dv;
  float* delta;
  const int32_t* hdr;
  const SeqInfo* seq;
  const int2* list;
  int32_t hq, hkv, group, d;
  float scale, scale_log2e;
};

}  // namespace attn
