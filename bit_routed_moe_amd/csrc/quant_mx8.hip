// MXFP8-E4M3 quantization of bf16 activation rows, the fp8 operand of the
// MXFP4 expert path on the scaled matrix instructions (the block rule is in
// formats.hpp).  A 32-value block is 64 bytes of bf16: four lanes take 16
// bytes each (coalesced), share the block's largest magnitude over two lane
// exchanges, and write 8 code bytes each; the block's first lane writes the
// scale byte.  Values come from bf16, so amax, the scale and value / scale are
// exact in fp32 and the one rounding is the E4M3 conversion.
#include "common.hpp"
#include "formats.hpp"
#include "launch.hpp"

namespace ds4 {

namespace {

__global__ __launch_bounds__(256) void mx8_quant_kernel(const uint16_t* __restrict__ x, int64_t nblk,
                                                        uint8_t* __restrict__ q, uint8_t* __restrict__ sc) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t blk = i >> 2;
    const int part = (int)(i & 3);
    const bool in = blk < nblk;   // the four lanes of a block agree
    u32x4 v = {0u, 0u, 0u, 0u};
    if (in) v = *reinterpret_cast<const u32x4*>(x + blk * 32 + part * 8);
    float f[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f[2 * j] = bf16_to_f32(v[j] & 0xFFFFu);
        f[2 * j + 1] = bf16_to_f32(v[j] >> 16);
    }
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(f[j]));
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    amax = fmaxf(amax, __shfl_xor(amax, 2));
    const uint32_t sb = mx8_scale_byte(amax);
    const float inv = mx8_inv_scale(sb);
    u32x2 o;
    o[0] = mx8_pack4(f[0] * inv, f[1] * inv, f[2] * inv, f[3] * inv);
    o[1] = mx8_pack4(f[4] * inv, f[5] * inv, f[6] * inv, f[7] * inv);
    if (in) {
        *reinterpret_cast<u32x2*>(q + blk * 32 + part * 8) = o;
        if (part == 0) sc[blk] = (uint8_t)sb;
    }
}

}  // namespace

hipError_t launch_quantize_mx8(const uint16_t* x, int64_t n, uint8_t* q, uint8_t* scales, hipStream_t s) {
    const int64_t nblk = n / 32;
    if (nblk == 0) return hipSuccess;
    const int64_t threads = nblk * 4;
    const int64_t grid = (threads + 255) / 256;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(mx8_quant_kernel, dim3((unsigned)grid), dim3(256), 0, s, x, nblk, q, scales);
    return hipGetLastError();
}

}  // namespace ds4
