// FP8 (E4M3) inputs of the forward: every E4M3 value (OCP 8-bit floating
// point: 1 sign, 4 exponent bits with bias 7, 3 mantissa bits, subnormals
// m * 2^-9, S.1111.111 NaN, no infinity) is exactly representable in bf16 and
// in fp16, so the codes are decoded exactly into 16-bit copies and the
// per-tensor descale factors are applied in the forward itself (scores and
// output).  TransformerEngine issue 2892 ("SIGSEGV in fused_attn_fwd when
// cu_seqlens_q != cu_seqlens_q_padded", section "Reproduction") runs this
// forward on THD inputs whose real boundaries differ from the padded ones.
#include "common.h"

namespace attn {

__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t e = (c >> 3) & 0xFu, m = c & 0x7u;
  float v;
  if (e == 0) v = (float)m * 0x1p-9f;                               // subnormal
  else v = __uint_as_float(((e + 120u) << 23) | (m << 20));          // 2^(e-7) (1 + m/8)
  if (e == 0xFu && m == 0x7u) v = __builtin_nanf("");
  return (c & 0x80u) ? -v : v;
}

// n codes (n % 8 == 0) -> n 16-bit values; 8 per thread, grid-stride.
template <int DT>
__global__ __launch_bounds__(256) void decode_e4m3_kernel(const uint8_t* __restrict__ src,
                                                          uint16_t* __restrict__ dst, int64_t n8) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (int64_t)gridDim.x * 256) {
    const u32x2 w = *reinterpret_cast<const u32x2*>(src + 8 * i);
    u32x4 o;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t x = w[h];
      o[2 * h] = Mfma<DT>::pack2(e4m3_to_f32(x & 0xFFu), e4m3_to_f32((x >> 8) & 0xFFu));
      o[2 * h + 1] = Mfma<DT>::pack2(e4m3_to_f32((x >> 16) & 0xFFu), e4m3_to_f32(x >> 24));
    }
    *reinterpret_cast<u32x4*>(dst + 8 * i) = o;
  }
}

hipError_t launch_decode_e4m3(const void* src, void* dst, int64_t n, int dtype, hipStream_t st) {
  const int64_t n8 = n / 8;
  if (n8 <= 0) return hipSuccess;
  const int64_t want = (n8 + 255) / 256;
  const unsigned grid = (unsigned)(want < 65536 ? want : 65536);
  if (dtype == kBF16)
    hipLaunchKernelGGL((decode_e4m3_kernel<kBF16>), dim3(grid), dim3(256), 0, st,
                       static_cast<const uint8_t*>(src), static_cast<uint16_t*>(dst), n8);
  else
    hipLaunchKernelGGL((decode_e4m3_kernel<kFP16>), dim3(grid), dim3(256), 0, st,
                       static_cast<const uint8_t*>(src), static_cast<uint16_t*>(dst), n8);
  return hipGetLastError();
}

}  // namespace attn
