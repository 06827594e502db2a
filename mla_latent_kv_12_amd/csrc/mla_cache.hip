// HIP kernel of the cache append of a decode step, written for gfx950.
//
// A decoded token's latent row is appended to the cache before attention
// reads it ("MLA & DSA 推理性能优化指南" §4, decode-flow figure: the output
// token goes into the cache), as one 576-value row [c_KV (512) | k_rope (64)]
// (§1.1 figure; §5.1: d_c = 512, d_rope = 64).  An fp8 cache stores a row as
// 576 e4m3fn bytes (§4.1 and §5.3: about 576 bytes per token) plus, in this
// library, one fp32 scale per token: scale = max|x| / 448 (1 for an all-zero
// row) and code = e4m3fn round-to-nearest-even of x / scale after clamping to
// +-448, all in fp32, so that e4m3fn(code) * scale is the stored value.
#include "mla_internal.h"

namespace mla {
namespace kern {

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr float kE4M3Max = 448.f;

__device__ __forceinline__ float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

// Eight bf16 values (one 16-byte piece) as fp32.
__device__ __forceinline__ void unpack8(const u32x4& v, float* x) {
#pragma unroll
  for (int i = 0; i < 4; i++) {
    x[2 * i] = bf16_lo(v[i]);
    x[2 * i + 1] = bf16_hi(v[i]);
  }
}

// Eight fp32 values divided by `scale`, clamped to +-448 and rounded to
// e4m3fn (the conversion rounds to nearest even), packed little-endian.
__device__ __forceinline__ u32x2 quant8(const float* x, float scale) {
  float q[8];
#pragma unroll
  for (int i = 0; i < 8; i++) q[i] = fminf(fmaxf(x[i] / scale, -kE4M3Max), kE4M3Max);
  int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
  w0 = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], w0, true);
  int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(q[4], q[5], 0, false);
  w1 = __builtin_amdgcn_cvt_pk_fp8_f32(q[6], q[7], w1, true);
  return u32x2{(unsigned)w0, (unsigned)w1};
}

// One wave per new row (b, s).  A row is 72 pieces of 16 bytes (8 bf16):
// lane l handles piece l, lanes 0..7 also piece 64 + l.
template <bool FP8>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= a.B * a.Sq) return;
  const int b = row / a.Sq, s = row - b * a.Sq;
  const int j = a.seqlens[b] - a.Sq + s;  // logical position of the new token
  if (j < 0) return;
  const int lp = j / kPage;
  if (lp >= a.bt_stride) return;
  const int pg = a.block_table[(size_t)b * a.bt_stride + lp];
  if (pg < 0 || pg >= a.num_pages) return;
  const size_t slot = (size_t)pg * kPage + (j % kPage);
  const u32x4* src = reinterpret_cast<const u32x4*>(a.src + (size_t)row * kD);
  const bool two = lane < 8;
  const u32x4 v0 = src[lane];
  const u32x4 v1 = two ? src[64 + lane] : u32x4{0u, 0u, 0u, 0u};
  if constexpr (!FP8) {
    u32x4* dst = reinterpret_cast<u32x4*>(a.kv + slot * (kD * 2));
    dst[lane] = v0;
    if (two) dst[64 + lane] = v1;
  } else {
    float x0[8], x1[8];
    unpack8(v0, x0);
    unpack8(v1, x1);  // zeros on lanes without a second piece
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 8; i++) m = fmaxf(m, fmaxf(fabsf(x0[i]), fabsf(x1[i])));
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    const float scale = m > 0.f ? m / kE4M3Max : 1.f;
    u32x2* dst = reinterpret_cast<u32x2*>(a.kv + slot * kD);
    dst[lane] = quant8(x0, scale);
    if (two) dst[64 + lane] = quant8(x1, scale);
    if (lane == 0) a.kv_scales[slot] = scale;
  }
}

}  // namespace
}  // namespace kern

hipError_t launch_append(const AppendArgs& a, bool fp8, hipStream_t stream) {
  const long long rows = (long long)a.B * a.Sq;
  const dim3 grid((unsigned)((rows + 3) / 4));
  if (fp8)
    hipLaunchKernelGGL(kern::append_kernel<true>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(kern::append_kernel<false>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
