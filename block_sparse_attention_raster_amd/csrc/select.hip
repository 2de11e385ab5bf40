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

__device__ __forceinline__ int wave_inclusive_scan(int x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x;
}

template <int D, int R>
__global__ __launch_bounds__(kSelThreads) void vsa_score_topk_kernel(VsaArgs a, const float* __restrict__ qbar,
                                                                     const float* __restrict__ kbar,
                                                                     int32_t* __restrict__ sel) {
  constexpr int DG = D / 4;                          // float4 groups per row
  constexpr int RPT = R / kSelWaves;                 // rows per thread
  constexpr int LPT = kColChunk * DG / kSelThreads;  // float4 loads per thread per chunk
  static_assert(R % kSelWaves == 0 && (kColChunk * DG) % kSelThreads == 0, "bad tiling");
  extern __shared__ __align__(16) unsigned char smem[];
  f32x4* qs = reinterpret_cast<f32x4*>(smem);                 // [R][DG]
  f32x4* ks = qs + R * DG;                                   // [DG][kColChunk], column swizzled
  uint32_t* hist = reinterpret_cast<uint32_t*>(ks + DG * kColChunk);  // [waves][256]
  uint32_t* sc = hist + kSelWaves * 256;                     // [R][nb]

  const int groups = (a.nq + R - 1) / R;
  const int bh = blockIdx.x / groups;
  const int row0 = (blockIdx.x - bh * groups) * R;
  const int nrows = min(R, a.nq - row0);
  const f32x4* qsrc = reinterpret_cast<const f32x4*>(qbar + ((int64_t)bh * a.nq + row0) * D);
  const f32x4* ksrc = reinterpret_cast<const f32x4*>(kbar + (int64_t)bh * a.nb * D);
  const int tid = threadIdx.x;

  for (int i = tid; i < R * DG; i += kSelThreads) qs[i] = (i < nrows * DG) ? qsrc[i] : f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- scores: thread (rg, col) computes rows rg*RPT .. rg*RPT+RPT-1 of one cube per chunk
  const int col = tid & (kColChunk - 1);
  const int rg = tid / kColChunk;
  f32x4 kreg[LPT];
  auto load_chunk = [&](int j0) {
#pragma unroll
    for (int m = 0; m < LPT; ++m) {
      const int i = tid + m * kSelThreads;
      const int dg = i % DG, j = i / DG;
      kreg[m] = (j0 + j < a.nb) ? ksrc[(int64_t)(j0 + j) * DG + dg] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  load_chunk(0);
  for (int j0 = 0; j0 < a.nb; j0 += kColChunk) {
    __syncthreads();
#pragma unroll
    for (int m = 0; m < LPT; ++m) {
      const int i = tid + m * kSelThreads;
      const int dg = i % DG, j = i / DG;
      ks[dg * kColChunk + (j ^ (dg & 15))] = kreg[m];
    }
    __syncthreads();
    if (j0 + kColChunk < a.nb) load_chunk(j0 + kColChunk);
    float acc[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) acc[i] = 0.f;
#pragma unroll 8
    for (int dg = 0; dg < DG; ++dg) {
      const f32x4 kv = ks[dg * kColChunk + (col ^ (dg & 15))];
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const f32x4 qv = qs[(rg * RPT + i) * DG + dg];
        acc[i] = fmaf(qv[0], kv[0], acc[i]);
        acc[i] = fmaf(qv[1], kv[1], acc[i]);
        acc[i] = fmaf(qv[2], kv[2], acc[i]);
        acc[i] = fmaf(qv[3], kv[3], acc[i]);
      }
    }
    if (j0 + col < a.nb) {
#pragma unroll
      for (int i = 0; i < RPT; ++i) sc[(rg * RPT + i) * a.nb + j0 + col] = orderable_key(acc[i]);
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
  return (size_t)a.select_rows * a.D * 4 + (size_t)kColChunk * a.D * 4 + (size_t)kSelWaves * 256 * 4 +
         (size_t)a.select_rows * a.nb * 4;
}

namespace {

template <int D, int R>
hipError_t launch_rows(const VsaArgs& a, const float* qbar, const float* kbar, int32_t* sel, size_t lds,
                       hipStream_t stream) {
  static std::atomic<int> raised{0};
  if (lds > 65536 && !raised.load(std::memory_order_acquire)) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&vsa_score_topk_kernel<D, R>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    raised.store(1, std::memory_order_release);
  }
  const int groups = (a.nq + R - 1) / R;
  hipLaunchKernelGGL((vsa_score_topk_kernel<D, R>), dim3(groups * a.B * a.Hh), dim3(kSelThreads), lds, stream,
                     a, qbar, kbar, sel);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const VsaArgs& a, const float* qbar, const float* kbar, int32_t* sel, size_t lds,
                    hipStream_t stream) {
  switch (a.select_rows) {
    case 4: return launch_rows<D, 4>(a, qbar, kbar, sel, lds, stream);
    case 8: return launch_rows<D, 8>(a, qbar, kbar, sel, lds, stream);
    case 16: return launch_rows<D, 16>(a, qbar, kbar, sel, lds, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t vsa_launch_score_topk(const VsaArgs& a, const float* qbar, const float* kbar, int32_t* sel,
                                 hipStream_t stream) {
  const size_t lds = vsa_select_lds_bytes(a);
  return a.D == 128 ? launch_d<128>(a, qbar, kbar, sel, lds, stream) : launch_d<64>(a, qbar, kbar, sel, lds, stream);
}
