// Block mean-pool (the "mean" of q and k per block that the block scores use;
// "FastVideo VSA" user guide, opening definition: every query block scores
// the key/value blocks). One workgroup pools one block of one (batch, head):
// q for every query block (prefix blocks and cubes) of q's grid, k for every
// cube of k's grid. Only
// the block's valid tokens are read and the sum is divided by their count.
// Reads go through the in-kernel index map, 16 bytes per lane; the sum is
// float32 and the result float32. Inputs are bf16 or fp16.

#include "vsa_device.h"

namespace {

constexpr int kPoolThreads = 256;

template <int D, bool F16>
__global__ __launch_bounds__(kPoolThreads) void vsa_pool_kernel(VsaArgs a, const __bf16* __restrict__ q,
                                                                const __bf16* __restrict__ k,
                                                                float* __restrict__ qbar,
                                                                float* __restrict__ kbar) {
  constexpr int CPR = D / 8;                 // 16-byte chunks per token row
  constexpr int RPP = kPoolThreads / CPR;    // rows per pass
  __shared__ float red[RPP][D + 4];

  const int per_head = a.nq + a.nb;
  const int bh = blockIdx.x / per_head;
  const int task = blockIdx.x - bh * per_head;
  const int b = bh / a.Hh, h = bh - b * a.Hh;
  const bool isq = task < a.nq;
  const VsaGrid& g = isq ? a.gq : a.gk;
  const int blk = isq ? task : a.gk.Pb + (task - a.nq);
  const __bf16* src = isq ? q + (int64_t)b * a.sb + (int64_t)h * a.sh : k + (int64_t)b * a.ksb + (int64_t)h * a.ksh;
  const int32_t sn = isq ? a.sn : a.ksn;
  float* dst = isq ? qbar + ((int64_t)bh * a.nq + task) * D
                   : kbar + ((int64_t)bh * a.nb + (task - a.nq)) * D;

  const BlockExt e = block_ext(g, blk);
  const int c = threadIdx.x % CPR;
  const int rsub = threadIdx.x / CPR;

  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;

#pragma unroll 4
  for (int r = rsub; r < e.n; r += RPP) {
    const int row = slot_row(g, e, r);
    const u32x4 x = *reinterpret_cast<const u32x4*>(src + (int64_t)row * sn + c * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (F16) {   // fp16 inputs (exact in float)
        acc[2 * i] += (float)__builtin_bit_cast(_Float16, (unsigned short)(x[i] & 0xFFFFu));
        acc[2 * i + 1] += (float)__builtin_bit_cast(_Float16, (unsigned short)(x[i] >> 16));
      } else {               // bf16: the upper half of a float
        acc[2 * i] += __uint_as_float(x[i] << 16);
        acc[2 * i + 1] += __uint_as_float(x[i] & 0xFFFF0000u);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) red[rsub][c * 8 + i] = acc[i];
  __syncthreads();
  if (threadIdx.x < D) {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < RPP; ++r) s += red[r][threadIdx.x];
    dst[threadIdx.x] = s / (float)e.n;
  }
}

}  // namespace

template <bool F16>
static void launch_pool(const VsaArgs& a, const void* q, const void* k, float* qbar, float* kbar, hipStream_t stream) {
  dim3 grid((a.nq + a.nb) * a.B * a.Hh);
  if (a.D == 128)
    hipLaunchKernelGGL((vsa_pool_kernel<128, F16>), grid, dim3(kPoolThreads), 0, stream, a, (const __bf16*)q,
                       (const __bf16*)k, qbar, kbar);
  else
    hipLaunchKernelGGL((vsa_pool_kernel<64, F16>), grid, dim3(kPoolThreads), 0, stream, a, (const __bf16*)q,
                       (const __bf16*)k, qbar, kbar);
}

hipError_t vsa_launch_pool(const VsaArgs& a, const void* q, const void* k, float* qbar, float* kbar,
                           hipStream_t stream) {
  if (a.f16) launch_pool<true>(a, q, k, qbar, kbar, stream);
  else launch_pool<false>(a, q, k, qbar, kbar, stream);
  return hipGetLastError();
}
