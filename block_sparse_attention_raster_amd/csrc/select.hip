// Block scores and per-row top-k, with the score rows held in LDS (fastbsa
// package page, section "How it works": selection stays on chip instead of
// writing the block-score matrix to HBM and running a separate top-k).
//
// A workgroup takes a group of query blocks of one (batch, head) and scores
// them against every cube, s[i][j] = qbar_i . kbar_j in float32 (the positive
// factor head_dim^-1/2 does not change the order and is left out). Each score
// is stored as an order-preserving 32-bit key in LDS; then one wave per row
// finds the topk-th largest key exactly by radix selection. Keys above it are
// kept; among keys equal to it the lowest cube ids are kept ("FastVideo VSA"
// user guide, section "Wan top-k behavior": top-k is the number of
// key/value blocks kept per query block). The kept ids are written in
// ascending order with a ballot prefix count, so the output is
// deterministic. Up to VSA_SELECT_MFMA_MAX_BLOCKS cubes the scores come from
// the fp32 matrix cores; beyond that from vector FMAs with LDS staging.

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

// Exact top-k of one row of order-preserving keys in LDS, by one wave; the
// ids go to out[0..topk) in ascending order. Keys are first offset by the
// row minimum and the radix digits start at the highest bit in which the
// offsets differ, so the first histogram spreads over the row's actual range
// instead of the few values the top byte of clustered scores takes.
__device__ __forceinline__ void row_topk(const uint32_t* s, int nb, int topk, uint32_t* wh, int lane,
                                         int32_t* out) {
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
  for (int j = lane; j < nb; j += 64) {
    const uint32_t key = s[j];
    mn = min(mn, key);
    mx = max(mx, key);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    mn = min(mn, (uint32_t)__shfl_xor((int)mn, o, 64));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, o, 64));
  }
  const uint32_t range = mx - mn;
  int hi = range ? 32 - __clz(range) : 0;  // offsets fit in `hi` bits
  uint32_t prefix = 0;                      // known bits of the wanted offset above `hi`
  int remaining = topk;                     // its rank among offsets matching the prefix
  while (hi > 0) {
    const int lo = hi > 8 ? hi - 8 : 0;
    const uint32_t dmask = (1u << (hi - lo)) - 1u;
#pragma unroll
    for (int i = 0; i < 4; ++i) wh[lane * 4 + i] = 0;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    for (int j = lane; j < nb; j += 64) {
      const uint32_t off = s[j] - mn;
      const uint32_t top = hi >= 32 ? 0u : (off >> hi);
      if (top == prefix) atomicAdd(&wh[(off >> lo) & dmask], 1u);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
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
    prefix = (prefix << (hi - lo)) | (uint32_t)digit;
    remaining -= above;
    hi = lo;
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
  }
  const uint32_t thr = mn + prefix;
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  int written = 0, eq_seen = 0;
  for (int j0 = 0; j0 < nb; j0 += 64) {
    const int j = j0 + lane;
    const uint32_t key = (j < nb) ? s[j] : 0u;
    const bool gt = (j < nb) && key > thr;
    const bool eq = (j < nb) && key == thr;
    const uint64_t eqm = __ballot(eq);
    const int eq_rank = eq_seen + __popcll(eqm & lt_mask);
    const bool take = gt || (eq && eq_rank < remaining);
    const uint64_t tm = __ballot(take);
    const int pos = written + __popcll(tm & lt_mask);
    if (take && pos < topk) out[pos] = j;
    written += __popcll(tm);
    eq_seen += __popcll(eqm);
  }
}

// row_topk with the row's keys held in registers: KPL keys per lane, key j
// of the row at lane j % 64, slot j / 64 (nb <= 64*KPL). The histogram
// passes then issue their LDS atomics back to back, with no reloads behind
// them.
template <int KPL>
__device__ __forceinline__ void row_topk_regs(const uint32_t* s, int nb, int topk, uint32_t* wh, int lane,
                                              int32_t* out) {
  uint32_t kr[KPL];
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const int j = lane + 64 * i;
    kr[i] = j < nb ? s[j] : 0u;
  }
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    if (lane + 64 * i < nb) {
      mn = min(mn, kr[i]);
      mx = max(mx, kr[i]);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    mn = min(mn, (uint32_t)__shfl_xor((int)mn, o, 64));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, o, 64));
  }
  const uint32_t range = mx - mn;
  int hi = range ? 32 - __clz(range) : 0;
  uint32_t prefix = 0;
  int remaining = topk;
  while (hi > 0) {
    const int lo = hi > 8 ? hi - 8 : 0;
    const uint32_t dmask = (1u << (hi - lo)) - 1u;
#pragma unroll
    for (int i = 0; i < 4; ++i) wh[lane * 4 + i] = 0;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      const uint32_t off = kr[i] - mn;
      const uint32_t top = hi >= 32 ? 0u : (off >> hi);
      if (lane + 64 * i < nb && top == prefix) atomicAdd(&wh[(off >> lo) & dmask], 1u);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
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
    prefix = (prefix << (hi - lo)) | (uint32_t)digit;
    remaining -= above;
    hi = lo;
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
  }
  const uint32_t thr = mn + prefix;
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  int written = 0, eq_seen = 0;
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const int j = lane + 64 * i;
    const bool in = j < nb;
    const bool gt = in && kr[i] > thr;
    const bool eq = in && kr[i] == thr;
    const uint64_t eqm = __ballot(eq);
    const int eq_rank = eq_seen + __popcll(eqm & lt_mask);
    const bool take = gt || (eq && eq_rank < remaining);
    const uint64_t tm = __ballot(take);
    const int pos = written + __popcll(tm & lt_mask);
    if (take && pos < topk) out[pos] = j;
    written += __popcll(tm);
    eq_seen += __popcll(eqm);
  }
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
  for (int r = wave; r < nrows; r += kSelWaves)
    row_topk(sc + r * a.nb, a.nb, a.topk, wh, lane, sel + ((int64_t)bh * a.nq + row0 + r) * a.topk);
}

// Scores on the fp32 matrix cores (v_mfma_f32_16x16x4f32) for up to
// VSA_SELECT_MFMA_MAX_BLOCKS cubes: one workgroup takes 16 query blocks of one head; each
// wave takes every eighth block of 16 cubes. In one MFMA step, lane group
// g = lane/16 contributes head-dim index 16*(c/4) + 4*g + c%4, so one
// 16-byte load instruction reads 64 contiguous bytes of each of 16 qbar or
// kbar rows, straight from global memory (L2-resident: workgroups of one
// head run on one XCD). The 16x16 result lands as keys in LDS;
// then each of the eight waves runs row_topk on two rows.
constexpr int kMfmaRows = 16;
constexpr int kMfmaWaves = 8;  // two rows per wave in the top-k phase

template <int D, int KPL>
__global__ __launch_bounds__(kMfmaWaves * 64) void vsa_score_topk_mfma_kernel(VsaArgs a, const float* __restrict__ qbar,
                                                                          const float* __restrict__ kbar,
                                                                          int32_t* __restrict__ sel) {
  constexpr int DQ = D / 4;
  extern __shared__ __align__(16) unsigned char smem[];
  uint32_t* sc = reinterpret_cast<uint32_t*>(smem);   // [16][nb]
  uint32_t* hist = sc + kMfmaRows * a.nb;               // [waves][256]

  const int groups = (a.nq + kMfmaRows - 1) / kMfmaRows;
  // XCD-aware order: consecutive workgroup ids go to different XCDs, so the
  // id is remapped to give each XCD a contiguous range (whole heads): a
  // head's kbar then stays in one XCD's L2
  const int nwg = groups * a.B * a.Hh;
  const int per_xcd = (nwg + 7) / 8;
  const int lid = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  if (lid >= nwg) return;
  const int bh = lid / groups;
  const int row0 = (lid - bh * groups) * kMfmaRows;
  const int nrows = min(kMfmaRows, a.nq - row0);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, l16 = lane & 15;

  float qv[DQ];
  {
    const bool ok = l16 < nrows;
    const f32x4* src = reinterpret_cast<const f32x4*>(qbar + ((int64_t)bh * a.nq + row0 + (ok ? l16 : 0)) * D + 4 * g);
#pragma unroll
    for (int i = 0; i < DQ / 4; ++i) {
      const f32x4 x = ok ? src[4 * i] : f32x4{0.f, 0.f, 0.f, 0.f};
      qv[4 * i] = x[0];
      qv[4 * i + 1] = x[1];
      qv[4 * i + 2] = x[2];
      qv[4 * i + 3] = x[3];
    }
  }
  const float* kbase = kbar + (int64_t)bh * a.nb * D + 4 * g;
  for (int cb = wave; cb * 16 < a.nb; cb += kMfmaWaves) {
    const int col = cb * 16 + l16;
    const bool ok = col < a.nb;
    const f32x4* src = reinterpret_cast<const f32x4*>(kbase + (int64_t)(ok ? col : 0) * D);
    float kv[DQ];
#pragma unroll
    for (int i = 0; i < DQ / 4; ++i) {
      const f32x4 x = ok ? src[4 * i] : f32x4{0.f, 0.f, 0.f, 0.f};
      kv[4 * i] = x[0];
      kv[4 * i + 1] = x[1];
      kv[4 * i + 2] = x[2];
      kv[4 * i + 3] = x[3];
    }
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < DQ; c += 2) {
      acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(qv[c], kv[c], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(qv[c + 1], kv[c + 1], acc1, 0, 0, 0);
    }
    if (ok) {
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[(4 * g + r) * a.nb + col] = orderable_key(acc0[r] + acc1[r]);
    }
  }
  __syncthreads();
  uint32_t* wh = hist + wave * 256;
  for (int r = wave; r < nrows; r += kMfmaWaves)
    row_topk_regs<KPL>(sc + r * a.nb, a.nb, a.topk, wh, lane, sel + ((int64_t)bh * a.nq + row0 + r) * a.topk);
}

}  // namespace

size_t vsa_select_lds_bytes(const VsaArgs& a) {
  if (a.nb <= VSA_SELECT_MFMA_MAX_BLOCKS) return (size_t)kMfmaRows * a.nb * 4 + (size_t)kMfmaWaves * 256 * 4;
  return (size_t)a.select_rows * a.D * 4 + (size_t)kColChunk * a.D * 4 + (size_t)kSelWaves * 256 * 4 +
         (size_t)a.select_rows * a.nb * 4;
}

namespace {

template <int D, int R>
hipError_t launch_rows(const VsaArgs& a, const float* qbar, const float* kbar, int32_t* sel, size_t lds,
                       hipStream_t stream) {
  static std::atomic<uint64_t> raised{0};
  if (lds > 65536) {
    const hipError_t e = vsa_raise_lds_limit(reinterpret_cast<const void*>(&vsa_score_topk_kernel<D, R>), raised);
    if (e != hipSuccess) return e;
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

template <int D, int KPL>
hipError_t launch_mfma_kpl(const VsaArgs& a, const float* qbar, const float* kbar, int32_t* sel, size_t lds,
                           hipStream_t stream) {
  static std::atomic<uint64_t> raised{0};
  if (lds > 65536) {
    const hipError_t e =
        vsa_raise_lds_limit(reinterpret_cast<const void*>(&vsa_score_topk_mfma_kernel<D, KPL>), raised);
    if (e != hipSuccess) return e;
  }
  const int groups = (a.nq + kMfmaRows - 1) / kMfmaRows;
  const int nwg = groups * a.B * a.Hh;
  hipLaunchKernelGGL((vsa_score_topk_mfma_kernel<D, KPL>), dim3((nwg + 7) / 8 * 8), dim3(kMfmaWaves * 64), lds,
                     stream, a, qbar, kbar, sel);
  return hipGetLastError();
}

// keys per lane of the register top-k: the next power of two >= nb / 64
template <int D>
hipError_t launch_mfma(const VsaArgs& a, const float* qbar, const float* kbar, int32_t* sel, size_t lds,
                       hipStream_t stream) {
  const int kpl = (a.nb + 63) / 64;
  if (kpl <= 2) return launch_mfma_kpl<D, 2>(a, qbar, kbar, sel, lds, stream);
  if (kpl <= 4) return launch_mfma_kpl<D, 4>(a, qbar, kbar, sel, lds, stream);
  if (kpl <= 8) return launch_mfma_kpl<D, 8>(a, qbar, kbar, sel, lds, stream);
  if (kpl <= 16) return launch_mfma_kpl<D, 16>(a, qbar, kbar, sel, lds, stream);
  return launch_mfma_kpl<D, 32>(a, qbar, kbar, sel, lds, stream);
}

}  // namespace

hipError_t vsa_launch_score_topk(const VsaArgs& a, const float* qbar, const float* kbar, int32_t* sel,
                                 hipStream_t stream) {
  const size_t lds = vsa_select_lds_bytes(a);
  if (a.nb <= VSA_SELECT_MFMA_MAX_BLOCKS)
    return a.D == 128 ? launch_mfma<128>(a, qbar, kbar, sel, lds, stream) : launch_mfma<64>(a, qbar, kbar, sel, lds, stream);
  return a.D == 128 ? launch_d<128>(a, qbar, kbar, sel, lds, stream) : launch_d<64>(a, qbar, kbar, sel, lds, stream);
}
