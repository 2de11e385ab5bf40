// Block scores and per-row top-k, with the score rows held in LDS (fastbsa
// package page, section "How it works": selection stays on chip instead of
// writing the block-score matrix to HBM and running a separate top-k).
//
// One workgroup takes R query blocks of one (batch, head). It scores them
// against every cube, s[i][j] = qbar_i . kbar_j in float32 (the positive
// factor head_dim^-1/2 does not change the order and is left out), stores
// each score as an order-preserving 32-bit key in LDS, and then one wave per
// row finds the topk-th largest key exactly with four 8-bit radix passes.
// Keys above it are kept; among keys equal to it the lowest cube ids are
// kept ("FastVideo VSA" user guide, section "Wan top-k behavior": top-k is
// the number of key/value blocks kept per query block). The kept ids are
// written in ascending order with a ballot prefix count, so the output is
// deterministic.

#include "vsa_device.h"
#include "vsa_limits.h"

#include <atomic>

namespace {

constexpr int kSelThreads = 256;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kColChunk = 64;   // cubes scored per LDS stage
constexpr int VSA_SELECT_ROWS_PER_THREAD = VSA_SELECT_MAX_ROWS / kSelWaves;

__device__ __forceinline__ int wave_inclusive_scan(int x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x;
}

template <int D>
__global__ __launch_bounds__(kSelThreads) void vsa_score_topk_kernel(VsaArgs a, const float* __restrict__ qbar,
                                                                     const float* __restrict__ kbar,
                                                                     int32_t* __restrict__ sel) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int R = a.select_rows;
  float* qs = reinterpret_cast<float*>(smem);                        // [R][D]
  float* ks = qs + R * D;                                            // [kColChunk][D + 1]
  uint32_t* hist = reinterpret_cast<uint32_t*>(ks + kColChunk * (D + 1));  // [waves][256]
  uint32_t* sc = hist + kSelWaves * 256;                             // [R][nb]

  const int groups = (a.nq + R - 1) / R;
  const int bh = blockIdx.x / groups;
  const int row0 = (blockIdx.x - bh * groups) * R;
  const int nrows = min(R, a.nq - row0);
  const float* qsrc = qbar + ((int64_t)bh * a.nq + row0) * D;
  const float* ksrc = kbar + (int64_t)bh * a.nb * D;
  const int tid = threadIdx.x;

  for (int i = tid; i < R * D; i += kSelThreads) qs[i] = (i < nrows * D) ? qsrc[i] : 0.f;

  // ---- scores: thread (rg, col) computes rows rg, rg+4, ... for one cube
  const int col = tid & (kColChunk - 1);
  const int rg = tid / kColChunk;
  for (int j0 = 0; j0 < a.nb; j0 += kColChunk) {
    __syncthreads();
    const int ncols = min(kColChunk, a.nb - j0);
    for (int i = tid; i < kColChunk * D; i += kSelThreads) {
      const int j = i / D, d = i - j * D;
      ks[j * (D + 1) + d] = (j < ncols) ? ksrc[(int64_t)(j0 + j) * D + d] : 0.f;
    }
    __syncthreads();
    float acc[VSA_SELECT_ROWS_PER_THREAD];
#pragma unroll
    for (int i = 0; i < VSA_SELECT_ROWS_PER_THREAD; ++i) acc[i] = 0.f;
    const float* kc = ks + col * (D + 1);
#pragma unroll 4
    for (int d = 0; d < D; d += 4) {
      const float k0 = kc[d], k1 = kc[d + 1], k2 = kc[d + 2], k3 = kc[d + 3];
#pragma unroll
      for (int i = 0; i < VSA_SELECT_ROWS_PER_THREAD; ++i) {
        const int r = rg + kSelWaves * i;
        if (r < R) {
          const f32x4 qv = *reinterpret_cast<const f32x4*>(qs + r * D + d);
          acc[i] = fmaf(qv[0], k0, acc[i]);
          acc[i] = fmaf(qv[1], k1, acc[i]);
          acc[i] = fmaf(qv[2], k2, acc[i]);
          acc[i] = fmaf(qv[3], k3, acc[i]);
        }
      }
    }
    if (col < ncols) {
#pragma unroll
      for (int i = 0; i < VSA_SELECT_ROWS_PER_THREAD; ++i) {
        const int r = rg + kSelWaves * i;
        if (r < R) sc[r * a.nb + j0 + col] = orderable_key(acc[i]);
      }
    }
  }
  __syncthreads();

  // ---- exact top-k per row, one wave per row
  const int wave = tid / 64, lane = tid & 63;
  uint32_t* wh = hist + wave * 256;
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  for (int r = wave; r < nrows; r += kSelWaves) {
    const uint32_t* s = sc + r * a.nb;
    uint32_t prefix = 0, pmask = 0;
    int remaining = a.topk;   // rank of the wanted key among keys matching the prefix
#pragma unroll 1
    for (int shift = 24; shift >= 0; shift -= 8) {
#pragma unroll
      for (int i = 0; i < 4; ++i) wh[lane * 4 + i] = 0;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      for (int j = lane; j < a.nb; j += 64) {
        const uint32_t key = s[j];
        if ((key & pmask) == prefix) atomicAdd(&wh[(key >> shift) & 255u], 1u);
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      __builtin_amdgcn_wave_barrier();
      // lane L holds bins 255-4L .. 252-4L, largest digit first
      int c[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) c[i] = (int)wh[255 - 4 * lane - i];
      const int tot = c[0] + c[1] + c[2] + c[3];
      const int incl = wave_inclusive_scan(tot, lane);
      const int excl = incl - tot;
      const uint64_t hit = __ballot(excl < remaining && remaining <= incl);
      const int src = __ffsll((unsigned long long)hit) - 1;
      int digit = 0, above = 0, cum = excl;
      bool found = false;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (!found && remaining <= cum + c[i]) {
          digit = 255 - 4 * lane - i;
          above = cum;
          found = true;
        }
        cum += c[i];
      }
      digit = __shfl(digit, src, 64);
      above = __shfl(above, src, 64);
      prefix |= (uint32_t)digit << shift;
      pmask |= 255u << shift;
      remaining -= above;
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      __builtin_amdgcn_wave_barrier();
    }
    // keys > prefix are kept; the first `remaining` keys == prefix are kept
    int32_t* out = sel + ((int64_t)bh * a.nq + row0 + r) * a.topk;
    int written = 0, eq_seen = 0;
    for (int j0 = 0; j0 < a.nb; j0 += 64) {
      const int j = j0 + lane;
      const uint32_t key = (j < a.nb) ? s[j] : 0u;
      const bool gt = (j < a.nb) && key > prefix;
      const bool eq = (j < a.nb) && key == prefix;
      const uint64_t eqm = __ballot(eq);
      const int eq_rank = eq_seen + __popcll(eqm & lt_mask);
      const bool take = gt || (eq && eq_rank < remaining);
      const uint64_t tm = __ballot(take);
      const int pos = written + __popcll(tm & lt_mask);
      if (take && pos < a.topk) out[pos] = j;
      written += __popcll(tm);
      eq_seen += __popcll(eqm);
    }
  }
}

}  // namespace

size_t vsa_select_lds_bytes(const VsaArgs& a) {
  return (size_t)a.select_rows * a.D * 4 + (size_t)kColChunk * (a.D + 1) * 4 +
         (size_t)kSelWaves * 256 * 4 + (size_t)a.select_rows * a.nb * 4;
}

// Lets the score/top-k kernels take more than 64 KiB of dynamic LDS.
hipError_t vsa_prepare_select(size_t lds_bytes) {
  static std::atomic<int> raised{0};
  if (lds_bytes <= 65536 || raised.load(std::memory_order_acquire)) return hipSuccess;
  const int cap = 160 * 1024;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&vsa_score_topk_kernel<128>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, cap);
  if (e == hipSuccess)
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&vsa_score_topk_kernel<64>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, cap);
  if (e == hipSuccess) raised.store(1, std::memory_order_release);
  return e;
}

hipError_t vsa_launch_score_topk(const VsaArgs& a, const float* qbar, const float* kbar, int32_t* sel,
                                 hipStream_t stream) {
  const int groups = (a.nq + a.select_rows - 1) / a.select_rows;
  dim3 grid(groups * a.B * a.Hh);
  const size_t lds = vsa_select_lds_bytes(a);
  if (a.D == 128)
    hipLaunchKernelGGL(vsa_score_topk_kernel<128>, grid, dim3(kSelThreads), lds, stream, a, qbar, kbar,
                       sel);
  else
    hipLaunchKernelGGL(vsa_score_topk_kernel<64>, grid, dim3(kSelThreads), lds, stream, a, qbar, kbar,
                       sel);
  return hipGetLastError();
}
