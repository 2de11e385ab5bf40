// Block scores and per-row top-k, with the score rows held in LDS (fastbsa
// package page, section "How it works": selection stays on chip instead of
// writing the block-score matrix to HBM and running a separate top-k).
//
// A workgroup takes a group of query blocks of one (batch, head) and scores
// them against every cube, s[i][j] = qbar_i . kbar_j in float32 (the positive
// factor head_dim^-1/2 does not change the order and is left out). Each score
// is stored as an order-preserving 32-bit key in LDS; then one wave per row
// finds the topk-th largest key exactly (a histogram over the row's score
// range, then the few keys of the bin that holds it ranked directly, with
// radix selection over the key bits as the general fallback). Keys above it are
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

// Cross-lane steps on the vector ALU (DPP row operations and the permlane
// swaps), with no LDS round trip.
template <int CTRL, int ROW_MASK = 0xF, bool ZERO_FILL = true>
__device__ __forceinline__ int dpp(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, ROW_MASK, 0xF, ZERO_FILL);
}
constexpr int kQuadXor1 = 0xB1, kQuadXor2 = 0x4E, kRowHalfMirror = 0x141, kRowMirror = 0x140;
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;

// x op'd over all 64 lanes, in every lane
template <typename Op>
__device__ __forceinline__ uint32_t wave_all(uint32_t x, Op op) {
  x = op(x, (uint32_t)dpp<kQuadXor1>((int)x));
  x = op(x, (uint32_t)dpp<kQuadXor2>((int)x));
  x = op(x, (uint32_t)dpp<kRowHalfMirror>((int)x));
  x = op(x, (uint32_t)dpp<kRowMirror>((int)x));
  const auto r16 = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = op(r16[0], r16[1]);
  const auto r32 = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return op(r32[0], r32[1]);
}
__device__ __forceinline__ uint32_t wave_min(uint32_t x) {
  return wave_all(x, [](uint32_t u, uint32_t v) { return u < v ? u : v; });
}
__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
  return wave_all(x, [](uint32_t u, uint32_t v) { return u > v ? u : v; });
}

// inclusive prefix sum over the 64 lanes: within each row of 16 lanes by
// shifts of 1, 2, 4 and 8, then the row totals carried across rows
__device__ __forceinline__ int wave_inclusive_scan(int x) {
  x += dpp<kRowShr1>(x);
  x += dpp<kRowShr2>(x);
  x += dpp<kRowShr4>(x);
  x += dpp<kRowShr8>(x);
  x += dpp<kRowBcast15, 0xA>(x);
  x += dpp<kRowBcast31, 0xC>(x);
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
  mn = wave_min(mn);
  mx = wave_max(mx);
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
    const int incl = wave_inclusive_scan(tot);
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
    digit = __builtin_amdgcn_readlane(digit, src);
    above = __builtin_amdgcn_readlane(above, src);
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
// passes issue their LDS atomics back to back, with no reloads behind them.
// After the first pass the bin that holds the topk-th key usually holds few
// keys; when it holds at most 64 they are gathered into one register per
// lane and the topk-th key is found among them directly (each candidate
// counts the candidates at or above it: the wanted key is the largest one
// with at least `remaining` of them), instead of by further passes. Both
// ways find the same key, and the final pass is shared.
// The float whose order-preserving key is k.
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Among the candidate keys `mine` (lanes < cnt, in no particular order),
// the largest key with at least `remaining` candidates at or above it.
// Returns it and lowers `remaining` by the candidates above it (leaving the
// number of keys equal to it still to take); `neq` is set to the whole
// number of keys equal to it.
__device__ __forceinline__ uint32_t rank_candidates(uint32_t mine, int cnt, int lane, int& remaining, int& neq) {
  int ge = 0;   // candidates at or above this lane's key
  for (int t = 0; t < cnt; ++t) ge += (uint32_t)__builtin_amdgcn_readlane((int)mine, t) >= mine;
  uint32_t cand = lane < cnt && ge >= remaining ? mine : 0u;
  cand = wave_max(cand);
  remaining -= __popcll(__ballot(lane < cnt && mine > cand));
  neq = __popcll(__ballot(lane < cnt && mine == cand));
  return cand;
}

// row_topk with the row's keys held in registers: KPL keys per lane, key j
// of the row at lane j % 64, slot j / 64 (nb <= 64*KPL). The first
// histogram spreads over the row's score range linearly: bin
// floor((x - min) * 256 / (max - min)) of the score x is monotone in x, so
// the bins above the one that holds the topk-th key hold exactly the keys
// greater than every key in it. That bin usually holds a few keys; when it
// holds at most 64 they are gathered into one register per lane and the
// topk-th key is found among them directly (each candidate counts the
// candidates at or above it: the wanted key is the largest one with at
// least `remaining` of them). Otherwise (many equal or clustered scores,
// or a range that is not finite) the keys are searched by radix selection
// over their bits, 8 at a time, from the highest bit in which the keys'
// offsets from the row minimum differ; its passes issue their LDS atomics
// back to back, and the same early exit applies after each pass. All ways
// find the same key, and the final pass is shared.
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
  mn = wave_min(mn);
  mx = wave_max(mx);
  const uint32_t range = mx - mn;
  int remaining = topk;      // rank of the wanted key among the keys still in play
  bool found_key = false;    // the wanted key is known (thr_direct)
  uint32_t thr_direct = 0;
  int neq = -1;              // keys equal to the wanted key, when known

  // the bin counts of this wave's histogram, read as four bins per lane from
  // the top, and the bin that holds the remaining-th key from the top: its
  // index, the keys above it and the keys in it
  auto find_bin = [&](int& digit, int& above, int& cnt) {
    int c[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = (int)wh[255 - 4 * lane - i];
    const int tot = c[0] + c[1] + c[2] + c[3];
    const int incl = wave_inclusive_scan(tot);
    const int excl = incl - tot;
    const uint64_t hit = __ballot(excl < remaining && remaining <= incl);
    const int src = __ffsll((unsigned long long)hit) - 1;
    int d = 0, ab = 0, cn = 0, cum = excl;
    bool found = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (!found && remaining <= cum + c[i]) {
        d = 255 - 4 * lane - i;
        ab = cum;
        cn = c[i];
        found = true;
      }
      cum += c[i];
    }
    digit = __builtin_amdgcn_readlane(d, src);
    above = __builtin_amdgcn_readlane(ab, src);
    cnt = __builtin_amdgcn_readlane(cn, src);
  };
  auto clear_hist = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) wh[lane * 4 + i] = 0;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
  };
  auto hist_done = [&]() {
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
  };
  // gather the keys for which `in(i)` holds (at most 64), one per lane, and
  // rank them
  auto gather_rank = [&](auto in, int cnt) {
    int base = 0;
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      const bool take = lane + 64 * i < nb && in(i);
      const uint64_t m = __ballot(take);
      if (take) wh[base + __popcll(m & ((1ull << lane) - 1ull))] = kr[i];
      base += __popcll(m);
    }
    hist_done();
    const uint32_t mine = lane < cnt ? wh[lane] : 0u;
    thr_direct = rank_candidates(mine, cnt, lane, remaining, neq);
    found_key = true;
    hist_done();
  };

  // linear first pass over the score values
  const float fmn = key_value(mn), fmx = key_value(mx);
  const float scale = 256.f / (fmx - fmn);
  if (range != 0u && __builtin_isfinite(fmn) && __builtin_isfinite(fmx) && __builtin_isfinite(scale) && scale > 0.f) {
    int bin[KPL];
#pragma unroll
    for (int i = 0; i < KPL; ++i)
      bin[i] = lane + 64 * i < nb ? min(255, (int)((key_value(kr[i]) - fmn) * scale)) : 0;
    clear_hist();
#pragma unroll
    for (int i = 0; i < KPL; ++i)
      if (lane + 64 * i < nb) atomicAdd(&wh[bin[i]], 1u);
    hist_done();
    int digit, above, cnt;
    find_bin(digit, above, cnt);
    hist_done();
    if (cnt <= 64) {
      remaining -= above;
      gather_rank([&](int i) { return bin[i] == digit; }, cnt);
    }
  }

  // radix selection over the key bits
  int hi = (found_key || range == 0u) ? 0 : 32 - __clz(range);   // offsets fit in `hi` bits
  uint32_t prefix = 0;   // known bits of the wanted offset above `hi`
  while (hi > 0) {
    const int lo = hi > 8 ? hi - 8 : 0;
    const uint32_t dmask = (1u << (hi - lo)) - 1u;
    clear_hist();
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      const uint32_t off = kr[i] - mn;
      const uint32_t top = hi >= 32 ? 0u : (off >> hi);
      if (lane + 64 * i < nb && top == prefix) atomicAdd(&wh[(off >> lo) & dmask], 1u);
    }
    hist_done();
    int digit, above, cnt;
    find_bin(digit, above, cnt);
    prefix = (prefix << (hi - lo)) | (uint32_t)digit;
    remaining -= above;
    hi = lo;
    hist_done();
    if (hi == 0) neq = cnt;   // the last digit's bin holds exactly the keys equal to it
    if (hi > 0 && cnt <= 64) {
      gather_rank([&](int i) { return ((kr[i] - mn) >> hi) == prefix; }, cnt);
      break;
    }
  }
  if (range == 0u) neq = nb;   // every key equals the row minimum
  const uint32_t thr = found_key ? thr_direct : mn + prefix;
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  int written = 0;
  if (neq == remaining) {
    // every key equal to the threshold is taken: the kept keys are those at
    // or above it
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      const int j = lane + 64 * i;
      const bool take = j < nb && kr[i] >= thr;
      const uint64_t tm = __ballot(take);
      const int pos = written + __popcll(tm & lt_mask);
      if (take && pos < topk) out[pos] = j;
      written += __popcll(tm);
    }
    return;
  }
  int eq_seen = 0;
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
// VSA_SELECT_MFMA_MAX_BLOCKS cubes: one workgroup of 8*RG waves takes 16*RG
// query blocks of one head, with their qbar rows in LDS; each wave takes
// every (8*RG)-th block of 16 cubes, loads its kbar rows straight from
// global memory (L2-resident: workgroups of one head run on one XCD) while
// the previous block's MFMAs run, and scores it against all RG groups of 16
// rows. In one MFMA step, lane group g = lane/16 contributes head-dim index
// 16*(c/4) + 4*g + c%4, so one 16-byte load reads 64 contiguous bytes of each
// of 16 kbar rows. Every workgroup streams the head's whole kbar through its
// CU, so two row groups halve that traffic; they need 32 score rows of LDS,
// which fit up to about a thousand cubes. The 16x16 results land as keys in
// LDS; then each wave runs row_topk on two rows.
template <int D, int KPL, int RG>
__global__ __launch_bounds__(RG * 8 * 64) void vsa_score_topk_mfma_kernel(VsaArgs a, const float* __restrict__ qbar,
                                                                          const float* __restrict__ kbar,
                                                                          int32_t* __restrict__ sel) {
  constexpr int kRows = 16 * RG, kWaves = 8 * RG;
  constexpr int DQ = D / 4;
  extern __shared__ __align__(16) unsigned char smem[];
  uint32_t* sc = reinterpret_cast<uint32_t*>(smem);   // [rows][nb]
  uint32_t* hist = sc + kRows * a.nb;                   // [waves][256]

  const int groups = (a.nq + kRows - 1) / kRows;
  // XCD-aware order: consecutive workgroup ids go to different XCDs, so the
  // id is remapped to give each XCD a contiguous range (whole heads): a
  // head's kbar then stays in one XCD's L2
  const int nwg = groups * a.B * a.Hh;
  const int per_xcd = (nwg + 7) / 8;
  const int lid = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  if (lid >= nwg) return;
  const int bh = lid / groups;
  const int row0 = (lid - bh * groups) * kRows;
  const int nrows = min(kRows, a.nq - row0);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, l16 = lane & 15;

  // the group's qbar rows in LDS, read per MFMA step
  f32x4* qs = reinterpret_cast<f32x4*>(hist + kWaves * 256);   // [rows][DQ]
  for (int i = tid; i < kRows * DQ; i += kWaves * 64) {
    const int r = i / DQ;
    qs[i] = r < nrows ? reinterpret_cast<const f32x4*>(qbar + ((int64_t)bh * a.nq + row0 + r) * D)[i - r * DQ]
                      : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  __syncthreads();
  const float* kbase = kbar + (int64_t)bh * a.nb * D + 4 * g;
  const int nblk = (a.nb + 15) / 16;
  auto load_block = [&](int cb, f32x4 (&kx)[DQ / 4]) {
    const int col = min(cb * 16 + l16, a.nb - 1);
    const f32x4* src = reinterpret_cast<const f32x4*>(kbase + (int64_t)col * D);
#pragma unroll
    for (int i = 0; i < DQ / 4; ++i) kx[i] = src[4 * i];
    __builtin_amdgcn_sched_barrier(0);   // issued before the MFMAs that follow
  };
  // one kbar block against every row group of the workgroup
  auto score_block = [&](int cb, const f32x4 (&kx)[DQ / 4]) {
    const int col = cb * 16 + l16;
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
      const f32x4* qrow = qs + (rg * 16 + l16) * DQ + g;   // quad 4i + g: head-dim 16i + 4g .. +3
      f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < DQ / 4; ++i) {
        const f32x4 qx = qrow[4 * i];
        acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(qx[0], kx[i][0], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(qx[1], kx[i][1], acc1, 0, 0, 0);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(qx[2], kx[i][2], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(qx[3], kx[i][3], acc1, 0, 0, 0);
      }
      if (col < a.nb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[(rg * 16 + 4 * g + r) * a.nb + col] = orderable_key(acc0[r] + acc1[r]);
      }
    }
  };
  f32x4 kb0[DQ / 4], kb1[DQ / 4];
  const int last = nblk - 1;
  if (wave < nblk) {
    load_block(wave, kb0);
    for (int cb = wave;;) {
      load_block(min(cb + kWaves, last), kb1);
      score_block(cb, kb0);
      cb += kWaves;
      if (cb >= nblk) break;
      load_block(min(cb + kWaves, last), kb0);
      score_block(cb, kb1);
      cb += kWaves;
      if (cb >= nblk) break;
    }
  }
  __syncthreads();
  uint32_t* wh = hist + wave * 256;
  for (int r = wave; r < nrows; r += kWaves)
    row_topk_regs<KPL>(sc + r * a.nb, a.nb, a.topk, wh, lane, sel + ((int64_t)bh * a.nq + row0 + r) * a.topk);
}

}  // namespace

namespace {

// LDS of the matrix-core kernel with RG groups of 16 rows: score rows,
// per-wave histograms and qbar rows
size_t mfma_lds_bytes(const VsaArgs& a, int rg) {
  return (size_t)16 * rg * a.nb * 4 + (size_t)8 * rg * 256 * 4 + (size_t)16 * rg * a.D * 4;
}

// Row groups per workgroup: two when their LDS fits and the launch still
// gives every CU a workgroup, else one.
int mfma_row_groups(const VsaArgs& a) {
  const int64_t wg2 = (int64_t)a.B * a.Hh * ((a.nq + 31) / 32);
  return mfma_lds_bytes(a, 2) <= 160 * 1024 && wg2 >= 256 ? 2 : 1;
}

}  // namespace

size_t vsa_select_lds_bytes(const VsaArgs& a) {
  if (a.nb <= VSA_SELECT_MFMA_MAX_BLOCKS) return mfma_lds_bytes(a, mfma_row_groups(a));
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

template <int D, int KPL, int RG>
hipError_t launch_mfma_kpl(const VsaArgs& a, const float* qbar, const float* kbar, int32_t* sel, size_t lds,
                           hipStream_t stream) {
  static std::atomic<uint64_t> raised{0};
  if (lds > 65536) {
    const hipError_t e =
        vsa_raise_lds_limit(reinterpret_cast<const void*>(&vsa_score_topk_mfma_kernel<D, KPL, RG>), raised);
    if (e != hipSuccess) return e;
  }
  const int groups = (a.nq + 16 * RG - 1) / (16 * RG);
  const int nwg = groups * a.B * a.Hh;
  hipLaunchKernelGGL((vsa_score_topk_mfma_kernel<D, KPL, RG>), dim3((nwg + 7) / 8 * 8), dim3(RG * 8 * 64), lds,
                     stream, a, qbar, kbar, sel);
  return hipGetLastError();
}

template <int D, int KPL>
hipError_t launch_mfma_rg(const VsaArgs& a, const float* qbar, const float* kbar, int32_t* sel, size_t lds,
                          hipStream_t stream) {
  return mfma_row_groups(a) == 2 ? launch_mfma_kpl<D, KPL, 2>(a, qbar, kbar, sel, lds, stream)
                                 : launch_mfma_kpl<D, KPL, 1>(a, qbar, kbar, sel, lds, stream);
}

// keys per lane of the register top-k: the next power of two >= nb / 64
template <int D>
hipError_t launch_mfma(const VsaArgs& a, const float* qbar, const float* kbar, int32_t* sel, size_t lds,
                       hipStream_t stream) {
  const int kpl = (a.nb + 63) / 64;
  if (kpl <= 2) return launch_mfma_rg<D, 2>(a, qbar, kbar, sel, lds, stream);
  if (kpl <= 4) return launch_mfma_rg<D, 4>(a, qbar, kbar, sel, lds, stream);
  if (kpl <= 8) return launch_mfma_rg<D, 8>(a, qbar, kbar, sel, lds, stream);
  if (kpl <= 16) return launch_mfma_rg<D, 16>(a, qbar, kbar, sel, lds, stream);
  return launch_mfma_rg<D, 32>(a, qbar, kbar, sel, lds, stream);
}

}  // namespace

hipError_t vsa_launch_score_topk(const VsaArgs& a, const float* qbar, const float* kbar, int32_t* sel,
                                 hipStream_t stream) {
  const size_t lds = vsa_select_lds_bytes(a);
  if (a.nb <= VSA_SELECT_MFMA_MAX_BLOCKS)
    return a.D == 128 ? launch_mfma<128>(a, qbar, kbar, sel, lds, stream) : launch_mfma<64>(a, qbar, kbar, sel, lds, stream);
  return a.D == 128 ? launch_d<128>(a, qbar, kbar, sel, lds, stream) : launch_d<64>(a, qbar, kbar, sel, lds, stream);
}
