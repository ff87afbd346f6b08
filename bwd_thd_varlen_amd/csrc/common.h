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
// 8*(u%2) + s: exactly a B (or A) operand in P-order.  The operand it meets
// must be read transposed from a row-major LDS tile in the same order; the
// gfx950 LDS transpose read does that (lds_tr_operand).
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
constexpr int kKVTile = 128;     // key rows per dK/dV work item
constexpr int kKVStep = 64;      // keys per inner step of dq_kernel (head dims up to 128)
constexpr int kMinTile = 64;     // smallest tile any list uses (sizes the lists)
constexpr int kSchedKeys = 2048; // distinct work keys of the heaviest-first ordering

// Workspace header (int32 words at the start of the workspace).
constexpr int kHdrStatus = 0;
constexpr int kHdrNQTiles = 1;
constexpr int kHdrNKVTiles = 2;
constexpr int kHdrWords = 64;    // 256 bytes

// Per-sequence record written by the scheduler.
// Token rows: token i of sequence b is row oq + i * ts of the q-side
// tensors (ok + i * ts on the kv side), with ts the layout's token stride:
// 1 for THD and bshd, the batch size for sbhd.
struct SeqInfo {
  int32_t oq, lq, ok, lk;        // first row of the slot and real lengths
  int32_t diag;                  // causal: key j is visible to query i iff j <= i + diag
};

// How token rows are laid out (the batched layouts have fixed slots of
// seqlen_q / seqlen_kv rows per sequence).
enum : int32_t { kLayoutThd = 0, kLayoutBshd = 1, kLayoutSbhd = 2 };

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
  // two stored values (low half first) widened to fp32, exactly
  static __device__ __forceinline__ f32x2 unpack2(uint32_t w) {
    return (f32x2){__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u)};
  }
};

// C += A B with E4M3 operands (OCP 8-bit floating point): the 32 x 32 x 64
// product; each operand is 32 codes per lane (row / column lane & 31, k range
// 32 (lane >> 5) .. +32) passed as two 16-byte halves; block scales 1.
__device__ __forceinline__ f32x16 mma_e4m3(u32x4 a0, u32x4 a1, u32x4 b0, u32x4 b1, f32x16 c) {
  typedef int v8i __attribute__((ext_vector_type(8)));
  const v8i a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                 (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
  const v8i b = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3],
                 (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

template <> struct Mfma<kFP16> {
  static __device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, f16x2));
  }
  static __device__ __forceinline__ f32x2 unpack2(uint32_t w) {
    return __builtin_convertvector(__builtin_bit_cast(f16x2, w), f32x2);
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

// ----------------------------------------------------------------- LDS tiles
// LDS tiles are row-major.  A row of DPAD 16-bit columns is padded by P
// 16-byte slots and stored shifted right by rot(r) slots, so element (r, c)
// sits at r * RE + 8 * rot(r) + c: offsets are linear in the column and,
// for rows 16 apart, in the row.  Every MFMA operand read is then a per-lane
// base plus an immediate offset (an XOR swizzle would need one address
// register per read; kept live across the loop, those spill).
//   Lay<DPAD, false> -- tiles read only by 16-byte row reads (lane l reads a
//     chunk of row base + (l & 31), 16 lanes per pass): P = 1, rot = 0; the
//     odd row stride (in 16-byte slots) puts 16 consecutive rows on 16
//     distinct bank groups.
//   Lay<DPAD, true> -- tiles also read transposed (ds_read_b64_tr_b16: 32
//     lanes per pass over 4 consecutive rows x 64 bytes): for DPAD >= 64,
//     P = 4 and rot = (r >> 2) & 3, free of bank conflicts for both reads
//     (64 banks of 4 bytes); DPAD = 32 keeps P = 1, rot = 0.
template <int DPAD, bool TR>
struct Lay {
  static constexpr bool ROT = TR && DPAD >= 64;
  static constexpr int P = ROT ? 4 : 1;
  static constexpr int CPR = DPAD / 8;          // data slots per row
  static constexpr int SPR = CPR + P;           // slots per row
  static constexpr int RE = 8 * SPR;            // elements per row
  static constexpr bool PADDED = true;
  static __device__ __forceinline__ int rot(int r) { return ROT ? ((r >> 2) & 3) : 0; }
  // logical chunk held by slot position `pos` of row r (-1: padding)
  static __device__ __forceinline__ int chunk_at(int r, int pos) {
    const int x = pos - rot(r);
    return (x >= 0 && x < CPR) ? x : -1;
  }
  static __device__ __forceinline__ int off(int r, int c) { return r * RE + 8 * rot(r) + c; }
  // 16-bit elements of a ROWS-row tile, rounded up to whole 1 KB DMA units
  template <int ROWS>
  static constexpr int elems() { return (ROWS * SPR + 63) / 64 * 512; }
};

// Unpadded alternative: the 16-byte chunks of row r are permuted by
// x -> x ^ swz(r) (conflict-free for row reads, transposed reads and whole-
// row staging); the smallest footprint and DMA count, but one address per
// (row block, chunk) pair.  Used where those addresses fit in registers.
template <int DPAD>
struct Swz {
  static constexpr int CPR = DPAD / 8;
  static constexpr int SPR = CPR;
  static constexpr int RE = DPAD;
  static constexpr bool PADDED = false;
  static __device__ __forceinline__ int swz(int r) {
    if constexpr (DPAD >= 128) return ((r & 3) << 2) | ((r >> 2) & 3);
    else if constexpr (DPAD == 64) return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
    else return (r >> 2) & 3;
  }
  // logical chunk held by slot position `pos` of row r (-1: padding)
  static __device__ __forceinline__ int chunk_at(int r, int pos) { return pos ^ swz(r); }
  static __device__ __forceinline__ int off(int r, int c) { return r * DPAD + (((c >> 3) ^ swz(r)) << 3) + (c & 7); }
  template <int ROWS>
  static constexpr int elems() { return (ROWS * SPR + 63) / 64 * 512; }
};

// 16-byte row read: columns [c, c+8) of row r (c a multiple of 8)
template <class L>
__device__ __forceinline__ u32x4 lds_row8(const uint16_t* tile, int r, int c) {
  return *reinterpret_cast<const u32x4*>(tile + L::off(r, c));
}

__device__ __forceinline__ u32x2 lds_tr4(const uint16_t* p) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// Transposed MFMA operand from a row-major tile, for a product that
// contracts over the tile's rows: lane l receives column 32*cb + (l & 31) at
// rows 16u + 8*(s/4) + 4*(l >> 5) + (s%4), s = 0..7 (the P-order of an
// accumulator tile).  ds_read_b64_tr_b16 hands lane i of each 16-lane group
// element (i & 3) of the 8-byte chunk addressed by lane 4k + (i >> 2), as its
// k-th value; so lane J of the group addresses row j0 + (J >> 2), columns
// c0 + 4*(J & 3) .. +3.
template <class L>
__device__ __forceinline__ u32x4 lds_tr_operand(const uint16_t* tile, int cb, int u, int lane) {
  const int J = lane & 15;
  const int c = 32 * cb + 16 * ((lane >> 4) & 1) + 4 * (J & 3);
  const int r = 16 * u + 4 * (lane >> 5) + (J >> 2);
  const u32x2 a = lds_tr4(tile + L::off(r, c));
  const u32x2 b = lds_tr4(tile + L::off(r + 8, c));
  u32x4 o = {a[0], a[1], b[0], b[1]};
  return o;
}

// Reads at an LDS byte address: 16 bytes, and the 8-byte transpose read.
__device__ __forceinline__ u32x4 lds_ld16(uint32_t a) {
  return *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(a);
}
__device__ __forceinline__ u32x2 lds_tr4_at(uint32_t a) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<__attribute__((address_space(3))) v4i16*>(a));
  return __builtin_bit_cast(u32x2, v);
}

// Operand readers for padded tiles (Lay): the lane-dependent part of every
// read's offset is formed once (one 32-bit LDS address per tile and step),
// and each read adds a compile-time constant, which goes into the
// instruction's offset field -- also when the tile is picked at run time
// from a ring.  `tile` is the tile's LDS byte address.
//   RowReader(tile, lane).read(rb, t): the 16-byte row read of lds_row8 at
//     row 32*rb + (lane & 31), columns 16*t + 8*(lane >> 5) ...
//   TrReader(tile, lane).read(cb, u): lds_tr_operand(tile, cb, u, lane).
template <class L>
struct RowReader {
  static_assert(L::PADDED, "linear offsets need the padded layout");
  uint32_t a;
  __device__ __forceinline__ RowReader(uint32_t tile, int lane)
      : a(tile + 2u * (uint32_t)L::off(lane & 31, 8 * (lane >> 5))) {}
  __device__ __forceinline__ u32x4 read(int rb, int t) const {
    return lds_ld16(a + 2u * (uint32_t)(32 * rb * L::RE + 16 * t));
  }
};
template <class L>
struct TrReader {
  static_assert(L::PADDED, "linear offsets need the padded layout");
  uint32_t a;
  __device__ __forceinline__ TrReader(uint32_t tile, int lane)
      : a(tile + 2u * (uint32_t)L::off(4 * (lane >> 5) + ((lane & 15) >> 2), 16 * ((lane >> 4) & 1) + 4 * (lane & 3))) {}
  __device__ __forceinline__ u32x4 read(int cb, int u) const {
    // rows r and r + 8 of the same lane: rot(r + 8) = rot(r) + 2 (r & 15 < 8)
    const uint32_t q = a + 2u * (uint32_t)(16 * u * L::RE + 32 * cb);
    const u32x2 x = lds_tr4_at(q);
    const u32x2 y = lds_tr4_at(q + 2u * (uint32_t)(8 * L::RE + (L::ROT ? 16 : 0)));
    u32x4 o = {x[0], x[1], y[0], y[1]};
    return o;
  }
};

// Operand readers for swizzled tiles (Swz), which hold one VGPR of
// lane-dependent address each.  The swizzle XORs a row's 16-byte chunk index
// with a function of the row's low four bits, and a row is a power of two
// bytes long, so for a fixed lane the chunk of k step t of a row read lies at
// base ^ 32 t bytes (chunk 2 t + hh), and that of column block cb of a
// transposed read at base ^ 64 cb (chunk 4 cb + w); rows 32 rb and 16 u on
// keep the swizzle and only add a constant.  One XOR per read replaces an
// address register per (k step, tile), which the compiler would otherwise
// hoist out of the loop.  `tile` is the tile's LDS byte address.
template <int DPAD>
struct SwzRowReader {   // = lds_row8<Swz<DPAD>>(tile, 32 rb + (lane & 31), 16 t + 8 (lane >> 5))
  static constexpr uint32_t RB = 2 * DPAD;   // bytes per row
  uint32_t base;
  __device__ __forceinline__ explicit SwzRowReader(int lane)
      : base(2u * (uint32_t)Swz<DPAD>::off(lane & 31, 8 * (lane >> 5))) {}
  // makes the base opaque, so that the per-read XORs stay in the loop
  __device__ __forceinline__ void refresh() { asm volatile("" : "+v"(base)); }
  __device__ __forceinline__ u32x4 read(uint32_t tile, int rb, int t) const {
    return lds_ld16(tile + 32u * RB * (uint32_t)rb + (base ^ (32u * (uint32_t)t)));
  }
};
template <int DPAD>
struct SwzTrReader {    // = lds_tr_operand<Swz<DPAD>>(tile, cb, u, lane)
  static constexpr uint32_t RB = 2 * DPAD;
  uint32_t b0, b8;      // rows r and r + 8 (their swizzles differ)
  __device__ __forceinline__ explicit SwzTrReader(int lane) {
    const int J = lane & 15;
    const int c = 16 * ((lane >> 4) & 1) + 4 * (J & 3);
    const int r = 4 * (lane >> 5) + (J >> 2);
    b0 = 2u * (uint32_t)Swz<DPAD>::off(r, c);
    b8 = 2u * (uint32_t)Swz<DPAD>::off(r + 8, c);
  }
  __device__ __forceinline__ void refresh() { asm volatile("" : "+v"(b0), "+v"(b8)); }
  __device__ __forceinline__ u32x4 read(uint32_t tile, int cb, int u) const {
    const uint32_t t = tile + 16u * RB * (uint32_t)u, x = 64u * (uint32_t)cb;
    const u32x2 a = lds_tr4_at(t + (b0 ^ x));
    const u32x2 b = lds_tr4_at(t + (b8 ^ x));
    u32x4 o = {a[0], a[1], b[0], b[1]};
    return o;
  }
};

// ----------------------------------------------------------------- LDS DMA
// Raw buffer resource over `bytes` bytes at p (no stride; the hardware range
// check returns zeros for any offset >= bytes and does not touch memory).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

constexpr uint32_t kOutOfRange = 0x80000000u;   // a lane offset the range check always rejects

// LDS byte address of a location in a __shared__ array.  For a static array
// (or an offset from one) this folds to a constant; callers that pick one of
// several buffers at run time add a byte offset to such a constant rather than
// converting a run-time pointer (that conversion costs a null test per use).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const void*)p);
}

// Global -> LDS DMA of BYTES (4 or 16) per lane: lane l's bytes land at
// lds_wave_base + BYTES * l (wave-uniform base); no VGPR is written.  Issued
// from inline asm so that the compiler does not try to order LDS reads
// against it (its alias tracking cannot tell the double buffers apart and
// would wait for the DMA of the next step); the kernels wait for their own
// DMA explicitly (wait_vm) and then barrier.  M0 is reserved by the
// compiler, but nothing else in these kernels uses it.
template <int BYTES>
__device__ __forceinline__ void dma(__amdgpu_buffer_rsrc_t rs, uint32_t lds_wave_base, uint32_t voff) {
  static_assert(BYTES == 4 || BYTES == 16, "4- or 16-byte lanes");
  const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_wave_base);
  if constexpr (BYTES == 16)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(lds), "v"(voff), "s"(rs) : "memory");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                 :: "s"(lds), "v"(voff), "s"(rs) : "memory");
}

// s_waitcnt for vector-memory operations only: at most n (< 64) outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait until at most k steps of STEP vector-memory operations each are
// outstanding (k is wave-uniform; s_waitcnt takes an immediate).
template <int STEP, int MAXK>
__device__ __forceinline__ void wait_vm_steps(int k) {
  static_assert(MAXK >= 0 && MAXK <= 4, "at most 4 steps in flight");
  if constexpr (MAXK >= 4) { if (k >= 4) { wait_vm<4 * STEP>(); return; } }
  if constexpr (MAXK >= 3) { if (k >= 3) { wait_vm<3 * STEP>(); return; } }
  if constexpr (MAXK >= 2) { if (k >= 2) { wait_vm<2 * STEP>(); return; } }
  if constexpr (MAXK >= 1) { if (k >= 1) { wait_vm<STEP>(); return; } }
  wait_vm<0>();
}

// Workgroup barrier for loops whose LDS is written only by DMA: the caller
// has already waited (wait_vm) for its own DMA, and every LDS read before the
// barrier has been consumed, so no memory fence is needed.  (A fenced
// __syncthreads would also wait for the DMA just issued for the next step.)
// The empty asm statements keep the compiler from moving memory accesses
// across the barrier.
__device__ __forceinline__ void barrier_lds_dma() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Workgroup barrier after LDS stores that other waves read next: waits for
// this wave's LDS operations only (lgkmcnt), not for its outstanding DMA
// (vmcnt), so a ring refill issued earlier keeps running across it.
__device__ __forceinline__ void barrier_lds_writes() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Fills a ROWS-row tile of layout L from global rows (row stride
// `rs_bytes`), NWAVES waves sharing the work.  Each 64-lane DMA instruction
// writes 1 KB of the tile, i.e. slots [64i, 64i + 64) of 16 bytes; slot s is
// row s / SPR, position s % SPR, which holds the data chunk L::chunk_at
// gives (none for a padding slot).  Padding slots, chunks at or beyond the head
// dim d and rows at or beyond the valid count come back as zeros.  When the
// instructions do not split evenly, a wave's extra instruction writes
// (zeros) to the 1 KB `sink` instead, so that every wave issues the same
// number of DMAs and can use the same wait count.
template <class L, int ROWS, int NWAVES>
struct TileDma {
  static constexpr int INSTR = (ROWS * L::SPR + 63) / 64;
  static constexpr int PER_WAVE = (INSTR + NWAVES - 1) / NWAVES;
  static constexpr bool SINK = PER_WAVE * NWAVES != INSTR;   // some wave issues a sink DMA
  uint32_t voff[PER_WAVE];

  __device__ __forceinline__ void init(int wave, int lane, int d, uint32_t rs_bytes) {
#pragma unroll
    for (int k = 0; k < PER_WAVE; ++k) {
      const int i = wave * PER_WAVE + k;
      const int slot = i * 64 + lane;
      const int r = slot / L::SPR;
      const int x = L::chunk_at(r, slot % L::SPR);
      // (all but the last test only matter for padded or unevenly split tiles)
      const bool ok = (!SINK || i < INSTR) && (ROWS * L::SPR % 64 == 0 || r < ROWS) &&
                      (!L::PADDED || x >= 0) && 8 * x < d;
      voff[k] = ok ? (uint32_t)r * rs_bytes + 16u * (uint32_t)x : kOutOfRange;
    }
  }
  // rows [0, rows_valid) of the tile start at `row0`; the tile and the sink
  // (1 KB, only used when SINK) are LDS byte addresses
  __device__ __forceinline__ void issue(const uint16_t* row0, int rows_valid, uint32_t rs_bytes,
                                        uint32_t tile, uint32_t sink, int wave) const {
    const int nr = __builtin_amdgcn_readfirstlane(rows_valid < 0 ? 0 : (rows_valid > ROWS ? ROWS : rows_valid));
    issue_rsrc(make_rsrc(row0, (uint32_t)nr * rs_bytes), tile, sink, wave);
  }
  __device__ __forceinline__ void issue_rsrc(__amdgpu_buffer_rsrc_t rsrc, uint32_t tile, uint32_t sink,
                                             int wave) const {
#pragma unroll
    for (int k = 0; k < PER_WAVE; ++k) {
      const int i = wave * PER_WAVE + k;
      dma<16>(rsrc, (!SINK || i < INSTR) ? tile + 1024u * (uint32_t)i : sink, voff[k]);
    }
  }
  // The same without the sink DMAs, for callers that wait for all of a
  // wave's outstanding DMAs (then the waves need not issue equal counts).
  __device__ __forceinline__ void issue_rsrc_exact(__amdgpu_buffer_rsrc_t rsrc, uint32_t tile, int wave) const {
#pragma unroll
    for (int k = 0; k < PER_WAVE; ++k) {
      const int i = wave * PER_WAVE + k;
      if (!SINK || i < INSTR) dma<16>(rsrc, tile + 1024u * (uint32_t)i, voff[k]);
    }
  }
  __device__ __forceinline__ void issue_exact(const uint16_t* row0, int rows_valid, uint32_t rs_bytes,
                                              uint32_t tile, int wave) const {
    const int nr = __builtin_amdgcn_readfirstlane(rows_valid < 0 ? 0 : (rows_valid > ROWS ? ROWS : rows_valid));
    issue_rsrc_exact(make_rsrc(row0, (uint32_t)nr * rs_bytes), tile, wave);
  }
};

// A value the compiler cannot prove wave-uniform (e.g. loaded by a vector
// load) but that is: keep it in a scalar register.
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Work item of a compute kernel: the (sequence, tile) pair and the
// sequence's record, all wave-uniform.
struct WorkItem {
  int b, tile;
  SeqInfo s;
};
__device__ __forceinline__ WorkItem load_item(const int2* list, const SeqInfo* seq, int item) {
  WorkItem w;
  const int2 e = list[item];
  w.b = uniform(e.x);
  w.tile = uniform(e.y);
  const SeqInfo s = seq[w.b];
  w.s.oq = uniform(s.oq);
  w.s.lq = uniform(s.lq);
  w.s.ok = uniform(s.ok);
  w.s.lk = uniform(s.lk);
  w.s.diag = uniform(s.diag);
  return w;
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

// Combine lanes l and l ^ 32 (the two half-waves) with the gfx950 half-wave
// swap, a VALU op, instead of an LDS permute.
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Maximum / sum of the N x 16 accumulator values of a lane as a balanced
// tree, so the reduction costs log depth rather than a 16N-long chain of
// dependent instructions.  The maximum goes three operands at a time (one
// v_max3 each).
template <int N>
__device__ __forceinline__ float tree_max(const f32x16 (&c)[N]) {
  constexpr int M = 16 * N;
  float t[M];
#pragma unroll
  for (int i = 0; i < M; ++i) t[i] = c[i / 16][i % 16];
  int n = M;
#pragma unroll
  for (int level = 0; level < 6; ++level) {
    if (n == 1) break;
    const int m = (n + 2) / 3;
#pragma unroll
    for (int i = 0; i < m; ++i) {
      float v = t[3 * i];
      if (3 * i + 1 < n) v = fmaxf(v, t[3 * i + 1]);
      if (3 * i + 2 < n) v = fmaxf(v, t[3 * i + 2]);
      t[i] = v;
    }
    n = m;
  }
  return t[0];
}
template <int N>
__device__ __forceinline__ float tree_sum(const f32x16 (&c)[N]) {
  float t[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    t[r] = c[0][r];
#pragma unroll
    for (int i = 1; i < N; ++i) t[r] += c[i][r];
  }
#pragma unroll
  for (int w = 8; w > 0; w >>= 1)
#pragma unroll
    for (int r = 0; r < w; ++r) t[r] += t[r + w];
  return t[0];
}

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
  int32_t causal;                // 0 none, 1 top-left, 2 bottom-right triangle
  const int32_t* q_pos0;         // top-left with chunk positions: diag = q_pos0 - kv_pos0
  const int32_t* kv_pos0;        // (either may be NULL = 0)
  int32_t layout;                // kLayoutThd: slots from the padded arrays;
  int32_t slot_q, slot_kv;       // batched layouts: fixed slot lengths
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
  int32_t layout, slot;          // token layout and (batched) slot length of this side
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
  float* delta;      // -Delta = -rowsum(dO o O), written by dQ's prologue
  float* lse2;       // LSE * log2(e), written by dQ's prologue
  const int32_t* hdr;
  const SeqInfo* seq;
  const int2* list;
  int32_t hq, hkv, group, d;
  // scale_log2e multiplies the scores; scale is the epilogue multiplier of dQ
  // and dK (the softmax scale, or for E4M3 inputs each kernel's own factor)
  float scale, scale_log2e;
  int32_t tsq, tskv;   // token strides in rows (1 for THD and bshd, batch for sbhd)
  int32_t accumulate;  // backward: bit kAccDq adds into dq, bit kAccDkDv into dk and dv
  // dropout: keep iff the element's random byte >= drop_t; kept values are
  // scaled by drop_scale = 256 / (256 - drop_t)
  uint32_t drop_t, seed_lo, seed_hi, drop_c3;   // drop_c3 = offset * hq
  float drop_scale;
  float out_scale;     // forward output multiplier (the V descale of FP8 inputs; else 1)
  // backward: Delta is formed times delta_scale (1; 1 / descale_v for E4M3
  // inputs, whose dS is then carried as dS / descale_v)
  float delta_scale;
  const void* q8;      // forward with E4M3 q and k (the scores on the 8-bit products)
  const void* k8;
  // dK/dV with a split GQA group: the query heads of a KV head are spread
  // over kv_split workgroups per key tile (kv_heads heads each), which write
  // fp32 partial dK (planes 0 .. kv_split-1 of part) and dV (planes kv_split
  // .. 2 kv_split-1), each plane part_plane floats laid out as dk; a second
  // kernel sums them in plane order
  int32_t kv_split, kv_heads;
  float* part;
  int64_t part_plane;
};
constexpr int32_t kAccDq = 1, kAccDkDv = 2;

// ----------------------------------------------------------------- dropout
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As
// Easy as 1, 2, 3", SC'11): ten rounds over a 4-word counter; each round
// forms the 64-bit products of words 0 and 2 with two constants and
// recombines their halves with words 1 and 3 and the key, which is bumped by
// two Weyl constants between rounds.  The key is wave-uniform (scalar adds).
__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                               uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0, p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    c0 = hi1 ^ c1 ^ k0;
    c1 = lo1;
    c2 = hi0 ^ c3 ^ k1;
    c3 = lo0;
  }
  return (u32x4){c0, c1, c2, c3};
}

// Keep mask of one 4 x 4 block of (query, key) positions of sequence b and
// query head h: one generator call with counter (key >> 2, query >> 2, b,
// offset * hq + h) and key (seed_lo, seed_hi); element (i, j) uses byte
// (j & 3) of word (i & 3).  Returns the four words.
__device__ __forceinline__ u32x4 dropout_block(const AttnParams& p, int b, int h, int i4, int j4) {
  return philox4x32_10((uint32_t)j4, (uint32_t)i4, (uint32_t)b, p.drop_c3 + (uint32_t)h,
                       p.seed_lo, p.seed_hi);
}
__device__ __forceinline__ bool keep_byte(uint32_t word, int byte, uint32_t t) {
  return ((word >> (8 * byte)) & 0xFFu) >= t;
}

// The four lanes of a quad (lanes 4k .. 4k+3) share their query quad in the
// forward and dQ kernels and their key quad in dK/dV, so each computes one of
// the four generator calls they all need and the words are exchanged.
// 4 x 4 word transpose across a quad: on entry lane c (= lane & 3) holds the
// four words of block c, on return word c of blocks 0..3 (slot g = block g).
// Swapping bit 0, then bit 1, between the lane index and the slot index moves
// every word to its transposed place; each swap sends two words per lane to
// the partner lane (DPP quad permutations [1,0,3,2] and [2,3,0,1]).
__device__ __forceinline__ u32x4 quad_transpose(const u32x4& m, int c) {
  const bool o0 = (c & 1) != 0, o1 = (c & 2) != 0;
  const uint32_t m0 = m.x, m1 = m.y, m2 = m.z, m3 = m.w;
  // bit 0: lanes with c odd send words 0 and 2 and take the partner's 1 and 3
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)(o0 ? m0 : m1), 0xB1, 0xF, 0xF, false);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)(o0 ? m2 : m3), 0xB1, 0xF, 0xF, false);
  const uint32_t n0 = o0 ? r0 : m0, n1 = o0 ? m1 : r0, n2 = o0 ? r1 : m2, n3 = o0 ? m3 : r1;
  // bit 1: lanes with c & 2 send words 0 and 1 and take the partner's 2 and 3
  const uint32_t t0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)(o1 ? n0 : n2), 0x4E, 0xF, 0xF, false);
  const uint32_t t1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)(o1 ? n1 : n3), 0x4E, 0xF, 0xF, false);
  return (u32x4){o1 ? t0 : n0, o1 ? t1 : n1, o1 ? n2 : t0, o1 ? n3 : t1};
}

// Byte transpose of a block's four words: word e of the result holds byte e
// of words 0..3, in that order (v_perm_b32 picks bytes of {hi, lo}: selector
// values 0-3 are lo's bytes, 4-7 hi's).  For the dK/dV kernels, whose lanes
// hold one key of every query row: after this and the quad transpose, slot g
// holds this lane's key byte of block g's four query rows.
__device__ __forceinline__ u32x4 byte_transpose(const u32x4& w) {
  const uint32_t a0 = __builtin_amdgcn_perm(w[1], w[0], 0x06020400u);
  const uint32_t a1 = __builtin_amdgcn_perm(w[1], w[0], 0x07030501u);
  const uint32_t a2 = __builtin_amdgcn_perm(w[3], w[2], 0x06020400u);
  const uint32_t a3 = __builtin_amdgcn_perm(w[3], w[2], 0x07030501u);
  return (u32x4){__builtin_amdgcn_perm(a2, a0, 0x05040100u), __builtin_amdgcn_perm(a3, a1, 0x05040100u),
                 __builtin_amdgcn_perm(a2, a0, 0x07060302u), __builtin_amdgcn_perm(a3, a1, 0x07060302u)};
}

// Applies the keep mask to the 16 values of this lane's query row in the four
// 4 x 4 blocks at key quads j4_0 + 2g (value 4g + e is key 4 (j4_0 + 2g) + e):
// dropped values become 0, kept ones are multiplied by `kept` (1, or the
// dropout scale).  Lane c of the quad computes block g = c; after the quad
// transpose slot g holds word c (this lane's query row) of block g.
__device__ __forceinline__ void dropout_row16(const AttnParams& p, int b, int h, int i4, int j4_0,
                                              int c, float kept, f32x16& v) {
  const u32x4 w = quad_transpose(dropout_block(p, b, h, i4, j4_0 + 2 * c), c);
  const uint32_t t = p.drop_t;
#define ATTN_DROP_APPLY(G, x)                                      \
  _Pragma("unroll") for (int e = 0; e < 4; ++e)                    \
      v[4 * G + e] = keep_byte(x, e, t) ? v[4 * G + e] * kept : 0.f;
  ATTN_DROP_APPLY(0, w.x)
  ATTN_DROP_APPLY(1, w.y)
  ATTN_DROP_APPLY(2, w.z)
  ATTN_DROP_APPLY(3, w.w)
#undef ATTN_DROP_APPLY
}

}  // namespace attn
