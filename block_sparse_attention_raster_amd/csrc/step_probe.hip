// Issue-rate, LDS-rate and synthetic-step probe for gfx950, run by the
// benchmark (`bench.py --step-probe`) as a child process; prints one JSON
// object. It measures what bounds the attention step's schedule rather than
// anything the attention computes:
//   - issue: cycles of exp2, fma and 32x32x16 bf16 MFMA mixes, one and two
//     waves per SIMD, independent chains (no dependency stalls);
//   - lds: bytes per clock per CU of conflict-free ds_read_b128 and
//     ds_read_b64_tr_b16 with two waves per SIMD, alone and beside MFMAs at
//     the attention step's ratio (one 1 KB operand read per MFMA);
//   - step: a synthetic attention step with the attention kernel's operand
//     shapes (64-key tile, head dim 128, K read four slots ahead, V four
//     slots ahead, the softmax's exp2 / pack / dot2 pipelined over the P.V
//     slots, P and the row sums used at the step's end as the row-sum check
//     uses them) but no global memory, walker or masking, then with a barrier
//     per two steps, with the step's global-to-LDS copies, and both; and the
//     same step with 64 query rows per wave at one wave per SIMD.
// Cycles come from s_memtime (the shader clock) per wave, median over waves.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdint>
#include <vector>

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kGrid = 256;           // one workgroup per CU
constexpr int kLdsBytes = 131072;    // dynamic LDS of every probe kernel
constexpr int kSrcBytes = 16 << 20;  // global source of the copies

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(size_t)((const __attribute__((address_space(3))) unsigned char*)p);
}
__device__ __forceinline__ u32x2 read_tr(uint32_t off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                       reinterpret_cast<__attribute__((address_space(3))) s16x4*>(off)));
}
__device__ __forceinline__ bf16x8 read_b128(const unsigned char* lds, uint32_t off) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(lds + off));
}
__device__ __forceinline__ void copy16(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "{m0}"(lds) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void record(long long* cyc, long long t0, long long t1) {
  if ((threadIdx.x & 63) == 0) cyc[blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64] = t1 - t0;
}

// ---- issue rates: per iteration two groups of (MFMA?) + NE exp2 + NF fma --
template <int NM, int NE, int NF>
__global__ void __launch_bounds__(512) issue_kernel(const float* __restrict__ in, float* __restrict__ sink,
                                                    long long* __restrict__ cyc, int iters) {
  const int tid = threadIdx.x;
  float a[8], b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = in[(tid + i) & 255];
    b[i] = in[(tid + 3 * i + 7) & 255];
  }
  const float c0 = in[300], c1 = in[301];
  bf16x8 x, y;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    x[i] = (__bf16)a[i];
    y[i] = (__bf16)b[i];
  }
  f32x16 acc0 = {}, acc1 = {};
  __syncthreads();
  const long long t0 = clock64();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      if constexpr (NM) {
        if (r == 0) acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, acc0, 0, 0, 0);
        else acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(y, x, acc1, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < NE; ++i) a[(r * NE + i) % 8] = __builtin_amdgcn_exp2f(a[(r * NE + i) % 8]);
#pragma unroll
      for (int i = 0; i < NF; ++i) b[(r * NF + i) % 8] = fmaf(b[(r * NF + i) % 8], c0, c1);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  const long long t1 = clock64();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += a[i] + b[i];
#pragma unroll
  for (int i = 0; i < 16; ++i) s += acc0[i] + acc1[i];
  sink[blockIdx.x * blockDim.x + tid] = s;
  record(cyc, t0, t1);
}

// ---- LDS read rates ------------------------------------------------------
// MODE 0: 8 ds_read_b128 per iteration; 1: 16 ds_read_b64_tr_b16; 2: two
// MFMAs with one b128 and two transposed reads (2 KB per wave).
template <int MODE>
__global__ void __launch_bounds__(512) lds_kernel(const unsigned* __restrict__ in, unsigned* __restrict__ sink,
                                                  long long* __restrict__ cyc, int iters) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < 65536 / 4; i += blockDim.x) reinterpret_cast<unsigned*>(lds)[i] = in[i & 255] + i;
  __syncthreads();
  u32x4 acc = {0, 0, 0, 0};
  f32x16 m0 = {}, m1 = {};
  bf16x8 x, y;
  for (int i = 0; i < 8; ++i) {
    x[i] = (__bf16)(float)(in[i] & 7);
    y[i] = (__bf16)(float)(in[i + 8] & 7);
  }
  // consecutive lanes read consecutive bytes: no bank conflicts; every
  // address stays below 64 KB
  const uint32_t b128 = (uint32_t)(wave * 4096 + lane * 16) & 65535;
  const uint32_t otr = (uint32_t)(wave * 4096 + lane * 8) & 65535;
  const uint32_t lds0 = lds_addr(lds);
  const long long t0 = clock64();
  for (int it = 0; it < iters; ++it) {
    if constexpr (MODE == 0) {
      u32x4 v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = *reinterpret_cast<const u32x4*>(lds + ((b128 + i * 1024) & 65535));
      asm volatile("" ::"v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7]));
    }
    if constexpr (MODE == 1) {
      u32x2 v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = read_tr(lds0 + ((otr + i * 512) & 65535));
      asm volatile("" ::"v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7]),
                   "v"(v[8]), "v"(v[9]), "v"(v[10]), "v"(v[11]), "v"(v[12]), "v"(v[13]), "v"(v[14]), "v"(v[15]));
    }
    if constexpr (MODE == 2) {
      const uint32_t o = (it & 7) * 512;
      const u32x4 v = *reinterpret_cast<const u32x4*>(lds + ((b128 + 2 * o) & 65535));
      const u32x2 w0 = read_tr(lds0 + ((otr + o) & 65535));
      const u32x2 w1 = read_tr(lds0 + ((otr + 2048 + o) & 65535));
      m0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, m0, 0, 0, 0);
      m1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(y, x, m1, 0, 0, 0);
      acc ^= v;
      acc.x ^= w0.x ^ w1.x;
      acc.y ^= w0.y ^ w1.y;
    }
    asm volatile("" ::: "memory");
  }
  const long long t1 = clock64();
  unsigned s = acc.x ^ acc.y ^ acc.z ^ acc.w;
  for (int i = 0; i < 16; ++i) s ^= __builtin_bit_cast(unsigned, m0[i] + m1[i]);
  sink[blockIdx.x * blockDim.x + tid] = s;
  record(cyc, t0, t1);
}

// ---- synthetic attention step ---------------------------------------------
// QB blocks of 32 query rows per wave; K ring and V ring of four 16 KB
// stages in LDS. BAR: one s_barrier per two steps; COPY: the step's copies
// (K of the tile two ahead, V of the tile one ahead, two 1 KB copies each
// per wave) from a 16 MB global buffer.
template <int QB, int NWAVE, bool BAR, bool COPY>
__global__ void __launch_bounds__(NWAVE * 64) step_kernel(const float* __restrict__ in, float* __restrict__ sink,
                                                          long long* __restrict__ cyc, int iters,
                                                          const unsigned char* __restrict__ src) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < kLdsBytes / 4; i += blockDim.x) reinterpret_cast<float*>(lds)[i] = in[i & 255] * 0.001f;
  __syncthreads();
  constexpr int NKB = 2, NC = 8, NQ = NKB * NC, NDB = 4, NP = NDB * 2 * NKB, NPAIR = NKB * 8, KA = 4, VRA = 4;
  bf16x8 qreg[QB][NC];
#pragma unroll
  for (int b = 0; b < QB; ++b)
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int i = 0; i < 8; ++i) qreg[b][c][i] = (__bf16)(in[(b * 64 + c * 8 + i + lane) & 255] * 0.01f);
  f32x16 oacc[QB][NDB], sa[QB][NKB];
  bf16x8 pb[QB][NKB][2];
  float ps[QB][4];
#pragma unroll
  for (int b = 0; b < QB; ++b) {
#pragma unroll
    for (int d = 0; d < NDB; ++d) oacc[b][d] = f32x16{};
#pragma unroll
    for (int k = 0; k < NKB; ++k) {
      sa[b][k] = f32x16{};
      pb[b][k][0] = bf16x8{};
      pb[b][k][1] = bf16x8{};
    }
    ps[b][0] = ps[b][1] = ps[b][2] = ps[b][3] = 0.f;
  }
  f32x16 negm;
#pragma unroll
  for (int i = 0; i < 16; ++i) negm[i] = -in[300];
  const bf16x2 one2 = {(__bf16)1.f, (__bf16)1.f};
  const uint32_t kbase = (uint32_t)lane * 16;             // K: 16 B per lane, conflict-free
  const uint32_t vbase = 65536u + (uint32_t)lane * 8;     // V: 8 B per lane
  const uint32_t lds0 = lds_addr(lds);
  __syncthreads();
  const long long t0 = clock64();
  for (int it = 0; it < iters; ++it) {
    const uint32_t kst = (it & 3) * 16384;
    const uint32_t vst = lds0 + vbase + (it & 3) * 16384;
    if constexpr (COPY) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t g = (uint32_t)(((it * 16 + wave * 2 + j) * 1024 + lane * 16) & (kSrcBytes - 1));
        copy16(src, g, lds0 + ((it + 2) & 3) * 16384 + (wave * 2 + j) * 1024);
        copy16(src, g ^ 0x80000u, lds0 + 65536 + ((it + 1) & 3) * 16384 + (wave * 2 + j) * 1024);
      }
    }
    bf16x8 kop[NQ];
    u32x4 vop[NP];
    auto vop_read = [&](int p) {
      const int ch = p / NDB, db = p % NDB;
      const u32x2 a0 = read_tr(vst + (db * 8 + 2 * ch) * 512), a1 = read_tr(vst + (db * 8 + 2 * ch + 1) * 512);
      vop[p] = u32x4{a0[0], a0[1], a1[0], a1[1]};
    };
#pragma unroll
    for (int i = 0; i < KA; ++i) kop[i] = read_b128(lds, kst + kbase + i * 1024);
#pragma unroll
    for (int qq = 0; qq < NQ; ++qq) {
      if (qq + KA < NQ) kop[qq + KA] = read_b128(lds, kst + kbase + (qq + KA) * 1024);
      if (qq >= NQ - VRA) vop_read(qq - (NQ - VRA));
      const int kb = qq / NC, c = qq % NC;
#pragma unroll
      for (int b = 0; b < QB; ++b)
        sa[b][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[qq], qreg[b][c], c != 0 ? sa[b][kb] : negm, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    f32x2 ex[QB][NPAIR];
    uint32_t wp[QB][NPAIR];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int ch = p / NDB, db = p % NDB;
      if (p + VRA < NP) vop_read(p + VRA);
#pragma unroll
      for (int b = 0; b < QB; ++b)
        oacc[b][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vop[p]),
                                                              pb[b][ch / 2][ch % 2], oacc[b][db], 0, 0, 0);
      // exp2 of pair p, packing of pair p-1, sum of pair p-2
#pragma unroll
      for (int b = 0; b < QB; ++b) {
        {
          const int kk = p, pkb = kk / 8, r = 8 * ((kk % 8) / 4) + 2 * (kk % 4);
          ex[b][kk] = f32x2{__builtin_amdgcn_exp2f(sa[b][pkb][r]), __builtin_amdgcn_exp2f(sa[b][pkb][r + 1])};
        }
        if (p >= 1) {
          const int kk = p - 1, pkb = kk / 8, phh = (kk % 8) / 4, i = kk % 4;
          const uint32_t w = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)ex[b][kk][0], (__bf16)ex[b][kk][1]});
          wp[b][kk] = w;
          if (i == 3)
            pb[b][pkb][phh] = __builtin_bit_cast(bf16x8, u32x4{wp[b][kk - 3], wp[b][kk - 2], wp[b][kk - 1], w});
        }
        if (p >= 2) {
          const int kk = p - 2;
          ps[b][kk % 4] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wp[b][kk]), one2, ps[b][kk % 4],
                                                         false);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      const int kk = NP - 1, pkb = kk / 8, phh = (kk % 8) / 4;
      const uint32_t w = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)ex[b][kk][0], (__bf16)ex[b][kk][1]});
      wp[b][kk] = w;
      pb[b][pkb][phh] = __builtin_bit_cast(bf16x8, u32x4{wp[b][kk - 3], wp[b][kk - 2], wp[b][kk - 1], w});
#pragma unroll
      for (int k2 = NP - 2; k2 < NP; ++k2)
        ps[b][k2 % 4] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wp[b][k2]), one2, ps[b][k2 % 4],
                                                       false);
    }
    // the step's P and sums are used here, as the attention kernel's row-sum
    // check uses them, so the compiler keeps the softmax inside the P.V slots
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      asm volatile("" ::"v"(pb[b][0][0]), "v"(pb[b][0][1]), "v"(pb[b][1][0]), "v"(pb[b][1][1]));
      asm volatile("" ::"v"(ps[b][0]), "v"(ps[b][1]), "v"(ps[b][2]), "v"(ps[b][3]));
    }
    if (it & 1) {
      if constexpr (COPY) wait_vmcnt<4>();   // copies of the step before have landed
      if constexpr (BAR) {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
      }
    }
  }
  const long long t1 = clock64();
  if constexpr (COPY) wait_vmcnt<0>();
  float s = 0.f;
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    s += ps[b][0] + ps[b][1] + ps[b][2] + ps[b][3];
#pragma unroll
    for (int d = 0; d < NDB; ++d)
#pragma unroll
      for (int i = 0; i < 16; ++i) s += oacc[b][d][i];
  }
  sink[blockIdx.x * blockDim.x + tid] = s;
  record(cyc, t0, t1);
}

struct Buffers {
  float* in = nullptr;
  float* sink = nullptr;
  long long* cyc = nullptr;
  unsigned char* src = nullptr;
};

bool check(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    fprintf(stderr, "step_probe: %s: %s\n", what, hipGetErrorString(e));
    return false;
  }
  return true;
}

// Median per-wave cycles of the second of two launches.
template <typename Launch>
bool median_cycles(const Buffers& bf, int waves_per_group, Launch launch, double* out) {
  launch();
  launch();
  if (!check(hipDeviceSynchronize(), "kernel")) return false;
  const int nw = kGrid * waves_per_group;
  std::vector<long long> c(nw);
  if (!check(hipMemcpy(c.data(), bf.cyc, nw * sizeof(long long), hipMemcpyDeviceToHost), "copy")) return false;
  std::sort(c.begin(), c.end());
  *out = (double)c[nw / 2];
  return true;
}

bool first = true;
void emit(const char* key, double v) {
  printf("%s\"%s\": %.1f", first ? "" : ", ", key, v);
  first = false;
}

template <int NM, int NE, int NF>
bool issue(const Buffers& bf, const char* key, int threads) {
  const int iters = 4096;
  double c;
  if (!median_cycles(bf, threads / 64, [&] {
        issue_kernel<NM, NE, NF><<<kGrid, threads>>>(bf.in, bf.sink, bf.cyc, iters);
      }, &c))
    return false;
  emit(key, c / iters);   // cycles per iteration (two groups) per wave
  return true;
}

template <int MODE>
bool lds_rate(const Buffers& bf, const char* key, double bytes_per_iter_wave) {
  const int iters = 4096, threads = 512;
  double c;
  if (!median_cycles(bf, threads / 64, [&] {
        lds_kernel<MODE><<<kGrid, threads, kLdsBytes>>>(reinterpret_cast<const unsigned*>(bf.in),
                                                          reinterpret_cast<unsigned*>(bf.sink), bf.cyc, iters);
      }, &c))
    return false;
  const double per_iter = c / iters;
  if (bytes_per_iter_wave > 0) emit(key, bytes_per_iter_wave * (threads / 64) / per_iter);   // B/clk/CU
  else emit(key, per_iter);
  return true;
}

template <int QB, int NWAVE, bool BAR, bool COPY>
bool step(const Buffers& bf, const char* key) {
  const int iters = 2048;
  double c;
  if (!median_cycles(bf, NWAVE, [&] {
        step_kernel<QB, NWAVE, BAR, COPY><<<kGrid, NWAVE * 64, kLdsBytes>>>(bf.in, bf.sink, bf.cyc, iters, bf.src);
      }, &c))
    return false;
  const double per_step = c / iters;
  const double mfma_cycles = 32.0 * 32.0 * QB * (NWAVE / 4);   // per SIMD per step
  emit(key, 100.0 * mfma_cycles / per_step);                   // MFMA busy %
  return true;
}

}  // namespace

int main() {
  Buffers bf;
  if (!check(hipMalloc(&bf.in, 1024 * sizeof(float)), "alloc") ||
      !check(hipMalloc(&bf.sink, kGrid * 1024 * sizeof(float)), "alloc") ||
      !check(hipMalloc(&bf.cyc, kGrid * 16 * sizeof(long long)), "alloc") ||
      !check(hipMalloc(&bf.src, kSrcBytes), "alloc") || !check(hipMemset(bf.src, 0x3c, kSrcBytes), "memset"))
    return 1;
  std::vector<float> h(1024);
  for (int i = 0; i < 1024; ++i) h[i] = -1.0f - (i % 7) * 0.1f;
  h[300] = 0.999f;   // fma multiplier and addend of the issue probe, the step's offset
  h[301] = 0.001f;
  if (!check(hipMemcpy(bf.in, h.data(), h.size() * sizeof(float), hipMemcpyHostToDevice), "copy")) return 1;
  printf("{");
  const bool ok =
      issue<0, 8, 0>(bf, "issue_exp16_1w", 256) && issue<0, 0, 8>(bf, "issue_fma16_1w", 256) &&
      issue<1, 0, 0>(bf, "issue_mfma2_1w", 256) && issue<0, 8, 0>(bf, "issue_exp16_2w", 512) &&
      issue<0, 0, 8>(bf, "issue_fma16_2w", 512) && issue<1, 0, 0>(bf, "issue_mfma2_2w", 512) &&
      issue<1, 1, 0>(bf, "issue_mfma2_exp2_2w", 512) && issue<1, 2, 0>(bf, "issue_mfma2_exp4_2w", 512) &&
      issue<1, 4, 0>(bf, "issue_mfma2_exp8_2w", 512) && issue<1, 0, 2>(bf, "issue_mfma2_fma4_2w", 512) &&
      issue<1, 0, 4>(bf, "issue_mfma2_fma8_2w", 512) && issue<1, 0, 8>(bf, "issue_mfma2_fma16_2w", 512) &&
      lds_rate<0>(bf, "lds_b128_bytes_per_clk_cu", 8 * 1024.0) &&
      lds_rate<1>(bf, "lds_tr_b64_bytes_per_clk_cu", 16 * 512.0) &&
      lds_rate<2>(bf, "lds_mfma2_read2k_cycles_2w", 0.0) &&
      step<1, 8, false, false>(bf, "step_mfma_busy_pct") && step<1, 8, true, false>(bf, "step_bar_mfma_busy_pct") &&
      step<1, 8, false, true>(bf, "step_copy_mfma_busy_pct") &&
      step<1, 8, true, true>(bf, "step_bar_copy_mfma_busy_pct") &&
      step<2, 4, false, false>(bf, "step_64rows_1w_mfma_busy_pct");
  printf("}\n");
  return ok ? 0 : 1;
}
