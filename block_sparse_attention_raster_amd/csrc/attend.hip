// Block-sparse flash attention over the kept blocks ("FastVideo VSA" user
// guide, opening definition: attention only against the selected top-k
// blocks; section "Choose top-k": prefix blocks are always kept; section
// "Verify routing and fallback": non-causal, scale head_size^-1/2).
//
// Work split. One workgroup owns RW = NW*32 query slots of one query block
// of one (batch, head); each wave owns 32 of them. The kept key blocks (all
// prefix blocks, then the selected cubes in ascending id order, cyclic from
// a start chosen per workgroup) are walked in tiles of KT key slots.
//
// Index map (fastbsa package page, section "How it works": the raster to
// block map is evaluated inside the kernel). The n valid tokens of a block
// are numbered k = (tt*eh + hh)*ew + ww over its valid extents (et, eh, ew)
// (partial cubes at the far edge of an axis have smaller extents); prefix
// block tokens are rows p*V + k. Both query rows and key tiles walk this
// compact numbering, so a block of n tokens fills floor(n/KT) whole key
// tiles and at most one tail tile. A tail tile's slots past n load the
// block's first row for K and zeros for V, so they need no masking: a
// correction after the step removes them from the row sum. The row offset
// (tt*H + hh)*W + ww of slot k depends only on the extents, which take four
// values per grid (whole or tail along h and along w), so the workgroup
// tabulates the four maps of the key grid (and the linear one of prefix
// blocks) at start-up as byte offsets, and each load reads its offset from
// LDS; query rows (read once) unravel k with multiply-high divisions. Query
// blocks follow q's grid and cube shape, key blocks k's (the two differ when
// q and k/v lie on different grids: fastbsa package page, section "Use").
// The workgroup also describes its kept blocks once, in walk order (the
// prefix blocks, then the selected cubes), in an LDS table, so moving from
// one kept block to the next costs one LDS read.
//
// Data movement. K and V tiles go from HBM straight into LDS with 16-byte
// copies that bypass registers (global_load_lds for K; buffer_load ... lds
// for V, through a buffer resource whose byte range ends at the head's
// last row, so that the out-of-range offset given to tail slots reads
// zeros) into two rings of NSTAGE tiles each. Step s reads K of tile s and
// V of tile s-1, so the copies of a tile's V are issued one step after its
// K: step s issues K of tile s+A and V of tile s+A-1, A = NSTAGE - BSTEP,
// into stages whose reads all finished before the last barrier. Each wave
// issues its share and waits for its own copies, and a barrier before every
// BSTEP-th step publishes them (BSTEP 2: one barrier per two tiles, with
// copies two tiles ahead in rings of four).
// Both tiles keep the natural [key][head_dim] order with the 16-byte chunks
// of each key row XOR-swizzled (applied on the global side, since the LDS
// position of each lane's 16 bytes is fixed by its lane id).
//
// MFMA mapping (v_mfma_f32_32x32x16_bf16, lanes l = 0..63, g = l / 32):
//   S^T = K Q^T : A = K rows (lane: key l%32, 8 head-dim values at 16c+8g),
//                 B = Q rows held in registers (lane: query l%32),
//                 C: lane holds query l%32, register r holds key
//                 8*(r/4) + 4*g + r%4.
//   O^T = V^T P^T: A = V^T (lane: head-dim l%32, 8 keys), B = P^T taken
//                 straight from the S^T accumulators (lane: query l%32),
//                 C: lane holds query l%32, register r holds head-dim
//                 8*(r/4) + 4*g + r%4.
// A lane feeds keys {4g..4g+3, 8+4g..8+4g+3} of a 16-key group to one P.V
// step; the matching V^T operand comes from two ds_read_b64_tr_b16 reads of
// the [key][head_dim] tile: in each 16-lane group, lane i addresses row
// key0 + i/4 at head-dim column base + 4*(i%4) and lane j receives the four
// keys key0..key0+3 of column base + j. Every lane owns one query row.
//
// Softmax in base 2 with a lazy offset: p = 2^x with x = c*s - m,
// c = head_dim^-1/2 * log2(e). For bf16 inputs the Q rows in registers are
// pre-multiplied by c (rounded once to bf16) and the first QK MFMA of each
// key block starts its accumulator at -m instead of 0, so the MFMA yields x
// and p = 2^x needs no further arithmetic. For fp16 inputs (held to a
// tighter tolerance) x = fma(s, c, -m) in fp32 instead, with Q unscaled.
// The offset m of a row is raised only when the
// tile's sum of p leaves a bound (so no p can exceed it): then the tile is
// redone with m raised to the row's maximum and O and l are rescaled. The
// first tile always sets m to its row maximum. Both O and l carry the same
// factor 2^-m, so this is the same softmax. The row sum adds p rounded to
// the input type (as P.V uses them) with v_dot2 against (1, 1).

#include <atomic>
#include <type_traits>

#include "vsa_device.h"
#include "vsa_limits.h"

namespace {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// The 16-bit element type of q, k, v, o and of P: bf16, or fp16 (the user
// guide's Wan route takes either, section "Verify routing and fallback").
// MFMA operands travel as raw 16-bit lanes (bf16x8 containers).
template <bool F16>
struct Elem {
  // two floats to one packed pair (round to nearest even)
  static __device__ __forceinline__ uint32_t pack2(float x, float y) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x, y}, bf16x2));
  }
  // the upper element of a packed pair, as float
  static __device__ __forceinline__ float hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
  // acc + both elements of a packed pair
  static __device__ __forceinline__ float sum2(uint32_t w, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), __builtin_bit_cast(bf16x2, 0x3F803F80u),
                                           acc, false);
  }
  static __device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // largest tile sum of p before the offset is raised (p <= this sum)
  static constexpr float kSumLimit = 16777216.f;  // 2^24
  // Q pre-scaled by c and the offset folded into the QK accumulators
  static constexpr bool kPrescale = true;
};
template <>
struct Elem<true> {
  static __device__ __forceinline__ uint32_t pack2(float x, float y) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x, y}, f16x2));
  }
  static __device__ __forceinline__ float sum2(uint32_t w, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w), __builtin_bit_cast(f16x2, 0x3C003C00u), acc, false);
  }
  // the upper element of a packed pair, as float
  static __device__ __forceinline__ float hi(uint32_t w) { return sum2(w & 0xFFFF0000u, 0.f); }
  static __device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
  }
  // fp16 P must stay below 65504
  static constexpr float kSumLimit = 32768.f;  // 2^15
  static constexpr bool kPrescale = false;
};

// The values of x held by lanes l % 32 and 32 + l % 32 (the two halves of a
// query row's keys), in every lane l: one v_permlane32_swap, which exchanges
// the upper half of its first operand with the lower half of its second.
__device__ __forceinline__ f32x2 halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return f32x2{__uint_as_float(r[0]), __uint_as_float(r[1])};
}

// Keeps x in a register at this point of the program (the compiler may not
// move its computation past here, nor fold it into later uses).
template <typename T>
__device__ __forceinline__ void pin(T& x) {
  asm volatile("" : "+v"(x));
}

// floor(x / d) for x, d < 2^16 with m = ceil(2^32 / d) (m = 2^32 for d = 1).
__device__ __forceinline__ int32_t fast_div(int32_t x, uint64_t m) {
  return (int32_t)(((uint64_t)(uint32_t)x * m) >> 32);
}

// Valid region of a kept or query block.
struct Blk {
  int32_t base;     // first token row (the row of index 0)
  int32_t n;        // valid tokens
  int32_t ew, ehw;  // valid extents ew and eh*ew (query rows unravel with them)
  uint64_t mw, mhw; // and their division magics
  int32_t type;     // video cubes: 2*[eh is the tail] + [ew is the tail]; prefix blocks 4
  bool prefix;
};

__device__ __forceinline__ Blk describe_block(const VsaGrid& g, int32_t blk) {
  Blk d;
  if (blk < g.Pb) {
    const int32_t s = blk * g.V;
    const int32_t n = min(g.V, g.P - s);
    d.base = s;
    d.n = n;
    d.ew = n;
    d.ehw = n;
    d.mw = d.mhw = 0;
    d.type = 4;
    d.prefix = true;
    return d;
  }
  const int32_t c = blk - g.Pb;
  const int32_t rest = fast_div(c, g.magic_nW);
  const int32_t bw = c - rest * g.nW;
  const int32_t bt = fast_div(rest, g.magic_nH);
  const int32_t bh = rest - bt * g.nH;
  const int32_t t0 = bt * g.ct, h0 = bh * g.ch, w0 = bw * g.cw;
  const int32_t et = min(g.ct, g.T - t0), eh = min(g.ch, g.H - h0), ew = min(g.cw, g.W - w0);
  const int ih = eh != g.ch, iw = ew != g.cw;
  d.base = g.P + (t0 * g.H + h0) * g.W + w0;
  d.n = et * eh * ew;
  d.ew = ew;
  d.ehw = eh * ew;
  d.mw = g.magic_ew[iw];
  d.mhw = g.magic_ehw[2 * ih + iw];
  d.type = 2 * ih + iw;
  d.prefix = false;
  return d;
}

// 16-byte global-to-LDS copies (global_load_lds_dwordx4: lane l's 16 bytes
// land at M0 + 16*l). Written as asm so that the compiler, which cannot tell
// these LDS writes apart from the kernel's LDS reads, does not make every LDS
// read wait for all copies in flight; the kernel orders them itself with
// explicit vmcnt waits and barriers. The compiler sets M0 from the input
// operand. No register outputs: nothing is written to VGPRs.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "{m0}"(lds) : "memory");
}
// The same through a buffer resource: a lane whose offset is past the
// resource's byte range (num_records) gets zeros, and no memory is read.
__device__ __forceinline__ void dma16_buf(i32x4 rsrc, uint32_t voff, uint32_t lds) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(lds) : "memory");
}

// Byte offset that is out of range of every V buffer resource (the plan
// keeps a head's K/V byte span at or below it).
constexpr uint32_t kOutOfRange = 0xFFFFFFC0u;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(size_t)((const __attribute__((address_space(3))) unsigned char*)p);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// LDS bytes of the slot tables: five maps of V_k entries plus KT entries of
// padding (a tile's slots past its block's end read there; their offsets
// are masked), rounded up to 16 bytes so that the kept-block table after
// them is aligned.
__host__ __device__ constexpr uint32_t slot_table_bytes(int32_t vk, int kt) {
  return ((uint32_t)(5 * vk + kt) * 4u + 15u) & ~15u;
}

template <int D, int NW, int NSTAGE, int KT, int WPE, bool F16, int BSTEP>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(WPE)))
void vsa_attend_kernel(VsaArgs a, const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                       const __bf16* __restrict__ v, const int32_t* __restrict__ sel, __bf16* __restrict__ o) {
  using E = Elem<F16>;
  constexpr int CPR = D / 8;             // 16-byte chunks per key row
  constexpr int NKB = KT / 32;           // 32-key MFMA blocks per tile
  constexpr uint64_t FULLM = KT == 64 ? ~0ull : ((1ull << (KT & 63)) - 1ull);
  static_assert(KT == 32 || KT == 64, "key tile of 32 or 64 slots");
  constexpr int RW = NW * 32;            // query slots per workgroup
  constexpr int UNITS = KT * CPR;        // 16-byte units per K (or V) tile
  constexpr int SLABS = UNITS / 64;      // wave-wide loads per tensor per tile
  constexpr int SPW = SLABS / NW;        // of which each wave issues
  constexpr int TILE_BYTES = UNITS * 16;
  constexpr int KSWZ = (CPR < 16 ? CPR : 16) - 1;
  static_assert(SLABS % NW == 0 && SPW >= 1, "tile loads must split evenly over the waves");
  static_assert(NSTAGE >= 2 && NSTAGE <= 4, "ring depth");
  constexpr int VM_PER_TILE = 2 * SPW;   // vector-memory instructions per wave per tile

  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* kst = smem;                              // [NSTAGE][TILE_BYTES]
  unsigned char* vst = smem + NSTAGE * TILE_BYTES;        // [NSTAGE][TILE_BYTES]
  const VsaGrid& gk = a.gk;     // key/value side
  // [5][V_k] (+ padding) byte offsets from a key block's first row of its
  // compact slots: video cubes by extent type (0..3), prefix blocks (4)
  uint32_t* stab = reinterpret_cast<uint32_t*>(smem + 2 * NSTAGE * TILE_BYTES);
  // [Pb + topk] kept blocks in walk order (prefix blocks, then the selected
  // cubes), as (first row's byte offset, n | slot-table base << 16)
  u32x2* blist = reinterpret_cast<u32x2*>(smem + 2 * NSTAGE * TILE_BYTES + slot_table_bytes(gk.V, KT));
  const uint32_t rowb = (uint32_t)a.ksn * 2u;   // bytes between key rows

  // XCD-aware order: consecutive workgroup ids go to different XCDs, so the
  // id is remapped to give each XCD a contiguous range of units (a unit is
  // RW query slots of one query block of one (batch, head)). The last
  // a.split_tail units of each range run as two workgroups of RW/2 slots
  // each (the other waves only load tiles): dispatched last, they shorten
  // the final, partly filled round of workgroups.
  const int nunits = a.B * a.Hh * a.nq * a.tiles;
  const int per_xcd = (nunits + 7) / 8;
  const int xcd = (int)(blockIdx.x % 8), jx = (int)(blockIdx.x / 8);
  const int nx = min(per_xcd, nunits - xcd * per_xcd);   // units of this XCD
  const int sx = min(a.split_tail, max(nx, 0));          // of which split
  int unit = xcd * per_xcd + jx, half = -1;              // half: -1 whole, else 0 or 1
  if (jx >= nx - sx) {
    const int hj = jx - (nx - sx);
    if (hj >= 2 * sx) return;
    unit = xcd * per_xcd + nx - sx + hj / 2;
    half = hj % 2;
  }
  int bid = unit;
  const int tile = bid % a.tiles;
  bid /= a.tiles;
  const int qblk = bid % a.nq;
  const int bh = bid / a.nq;
  const int b = bh / a.Hh, h = bh - b * a.Hh;
  const Blk qd = describe_block(a.gq, qblk);
  const int slot0 = tile * RW + (half > 0 ? RW / 2 : 0);
  const int rows_here = half < 0 ? RW : RW / 2;   // query slots of this workgroup
  if (slot0 >= qd.n) return;

  // Walk phase. The selected cubes are visited in ascending id order from a
  // starting position rot, cyclically. With many small workgroups resident
  // per XCD, a workgroup starts whenever an earlier one ends, so in steady
  // state the resident set started at staggered times; a start position
  // proportional to the dispatch index within a period of about the resident
  // set's size (walk_conc) keeps the cubes being read at any moment within a
  // narrow band of cube ids, which the XCD's L2 then holds. The order only changes float rounding, and it
  // depends on the launch alone, so results stay reproducible.
  const int rot = a.walk_conc > 0
                      ? (int)((int64_t)((blockIdx.x / 8) % (uint32_t)a.walk_conc) * a.topk / a.walk_conc)
                      : 0;

  const int tid = threadIdx.x;
  {  // Byte offsets from a key block's first row of its compact slots s:
     // for the four cube extent types (eh, ew) in {ch, tail} x {cw, tail},
     // slot s is (tt, hh, ww) in raster order over the valid extents; prefix
     // blocks are contiguous. Entries past a block's token count are never
     // used for a valid slot.
    const int tail_h = gk.H - (gk.nH - 1) * gk.ch, tail_w = gk.W - (gk.nW - 1) * gk.cw;
    for (int idx = tid; idx < 5 * gk.V + KT; idx += NW * 64) {
      const int t = idx / gk.V, s = idx - t * gk.V;
      int row = s;
      if (t < 4) {
        const int eh = (t >> 1) ? tail_h : gk.ch, ew = (t & 1) ? tail_w : gk.cw;
        const int ehw = eh * ew;
        const int tt = s / ehw, r = s - tt * ehw;
        const int hh = r / ew, ww = r - hh * ew;
        row = (tt * gk.H + hh) * gk.W + ww;
      }
      stab[idx] = t < 5 ? (uint32_t)row * rowb : 0u;
    }
    // the prefix blocks, then the selected cubes in walk order (ids clamped
    // into range: other contents of sel stay in bounds)
    const int32_t* selrow = sel + ((int64_t)(b * a.Hh + h) * a.nq + qblk) * a.topk;
    for (int i = tid; i < gk.Pb + a.topk; i += NW * 64) {
      int blk = i;
      if (i >= gk.Pb) {
        int t = i - gk.Pb + rot;
        if (t >= a.topk) t -= a.topk;
        int c = selrow[t];
        c = c < 0 ? 0 : (c >= a.nb ? a.nb - 1 : c);
        blk = gk.Pb + c;
      }
      const Blk d = describe_block(gk, blk);
      blist[i] = u32x2{(uint32_t)d.base * rowb, (uint32_t)d.n | ((uint32_t)(d.type * gk.V) << 16)};
    }
  }
  __syncthreads();

  const __bf16* qh = q + (int64_t)b * a.sb + (int64_t)h * a.sh;
  const int64_t kv_off = (int64_t)b * a.ksb + (int64_t)h * a.ksh;
  const __bf16* kh = k + kv_off;
  const __bf16* vh = v + kv_off;
  __bf16* oh = o + (int64_t)b * a.osb + (int64_t)h * a.osh;

  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int l32 = lane & 31, g = lane >> 5;

  // token row of compact index k < d.n of the query block (q's grid; every
  // video cube, whole or partial, carries its extents' division magics)
  auto query_row = [&](const Blk& d, int kk) -> int {
    if (d.prefix) return d.base + kk;
    const int tt = fast_div(kk, d.mhw);
    const int r = kk - tt * d.ehw;
    const int hh = fast_div(r, d.mw);
    const int ww = r - hh * d.ew;
    return d.base + (tt * a.gq.H + hh) * a.gq.W + ww;
  };

  // ---- Q row of this lane in MFMA B-operand layout (for bf16 scaled by
  // c = head_dim^-1/2 log2(e))
  const float cexp = a.scale_log2e;
  int qrow;
  bf16x8 qreg[D / 16];
  {
    const int rel = wave * 32;
    const int slot = slot0 + rel + l32;
    qrow = slot < qd.n && rel < rows_here ? query_row(qd, slot) : -1;
    if (qrow >= 0) {
      const __bf16* src = qh + (int64_t)qrow * a.sn + 8 * g;
#pragma unroll
      for (int c = 0; c < D / 16; ++c) qreg[c] = *reinterpret_cast<const bf16x8*>(src + 16 * c);
    } else {
#pragma unroll
      for (int c = 0; c < D / 16; ++c) qreg[c] = bf16x8{};
    }
  }
  // Q must be resident before the tile loads start: inside the loop the
  // compiler cannot count how many later loads follow it and would otherwise
  // wait for all of them before every tile.
  wait_vmcnt<0>();
  if constexpr (E::kPrescale) {
    static_assert(!F16, "the pre-scaled Q rows are bf16");
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      u32x4 w = __builtin_bit_cast(u32x4, qreg[c]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = E::pack2(__uint_as_float(w[i] << 16) * cexp, __uint_as_float(w[i] & 0xFFFF0000u) * cexp);
      qreg[c] = __builtin_bit_cast(bf16x8, w);
    }
  }
  const bool wave_active = __ballot(qrow >= 0) != 0;

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
  float lrow = 0.f;               // this lane's part of the row sum l
  float mneg = 0.f;               // -m (both lanes of a row agree)
  f32x16 negm = {};               // -m in every entry: with kPrescale the QK accumulators start there

  // ---- kept-block walk (issue side) over the LDS table: all prefix blocks
  // of the key grid, then the selected cubes
  const int nkept = gk.Pb + a.topk;
  int ibi = 0;        // current kept block
  int kt0 = 0;        // compact index of its next tile's first slot
  uint32_t kbase = 0; // its first row's byte offset
  int kn = 0;         // its valid tokens
  int ktab = 0;       // its slot-table base (extent type * V_k)
  u32x2 nxt;          // table entry of the block after it (an LDS read in flight)
  auto fetch = [&](int i) { nxt = blist[min(i, nkept - 1)]; };
  // the block whose table entry nxt holds
  auto next_block = [&](uint32_t& base, int& n, int& tab) {
    const uint32_t e0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)nxt[0]);
    const uint32_t e1 = (uint32_t)__builtin_amdgcn_readfirstlane((int)nxt[1]);
    base = e0;
    n = (int)(e1 & 0xFFFFu);
    tab = (int)(e1 >> 16);
  };
  fetch(0);
  next_block(kbase, kn, ktab);
  fetch(1);
  // bound of every K load's row offset, and the V buffer resource: V of
  // this head, num_records = its byte span, so that offsets at or past it
  // (tail slots) read as zeros
  const uint32_t last_b = (uint32_t)(gk.P + gk.T * gk.H * gk.W - 1) * rowb;
  i32x4 vrsrc;
  {
    const uint64_t vb = (uint64_t)reinterpret_cast<uintptr_t>(vh);
    vrsrc[0] = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)vb);
    vrsrc[1] = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)((vb >> 32) & 0xFFFFu));
    vrsrc[2] = __builtin_amdgcn_readfirstlane((int32_t)(last_b + (uint32_t)D * 2u));
    vrsrc[3] = 0x00020000;
  }

  // One tile of the walk: the block's first row, the valid slots from the
  // tile on (KT or more: all; 0 past the walk) and the slot-table index of
  // its first slot.
  struct Spec {
    uint32_t base;
    int32_t nleft;
    int32_t tk0;
  };
  struct Pend {
    uint32_t ko[SPW];  // K byte offsets from kh
    uint32_t vo[SPW];  // V byte offsets from vh (out of range for tail slots)
  };
  // describes the walker's current tile, then advances (branch-free: the
  // values are wave-uniform and selected, and the table entry of the block
  // after the current one is read one call ahead)
  auto spec = [&](Spec& sp, uint64_t& m, bool& e) {
    const bool any = ibi < nkept;
    const int nleft = any ? kn - kt0 : 0;
    sp.base = any ? kbase : 0u;
    sp.nleft = nleft;
    sp.tk0 = ktab + kt0;
    e = any;
    m = nleft >= KT ? FULLM : ((1ull << nleft) - 1ull);
    const bool adv = any && nleft <= KT;   // this tile ends its block
    uint32_t nbase;
    int nn, ntab;
    next_block(nbase, nn, ntab);
    kbase = adv ? nbase : kbase;
    kn = adv ? nn : kn;
    ktab = adv ? ntab : ktab;
    kt0 = adv ? 0 : (any ? kt0 + KT : kt0);
    ibi = adv ? ibi + 1 : ibi;
    fetch(ibi + 1);
  };

  // Thread (wave, lane) loads 16-byte unit s*64 + lane of each K and V tile
  // for s = wave*SPW + j: key row (s*64 + lane)/CPR, chunk position
  // (s*64 + lane)%CPR, XOR-swizzled by key (K: chunk ^ (key & KSWZ); V: see
  // the transposed reads).
  int keyj[SPW];
  uint32_t kcst[SPW], vcst[SPW];
#pragma unroll
  for (int j = 0; j < SPW; ++j) {
    const int p = (wave * SPW + j) * 64 + lane;
    const int key = p / CPR, cp = p % CPR;
    const int fv = (D == 128) ? 4 * (key & 3) : 4 * ((key >> 1) & 1);
    keyj[j] = key;
    kcst[j] = (uint32_t)((cp ^ (key & KSWZ)) * 16);
    vcst[j] = (uint32_t)((cp ^ fv) * 16);
  }
  // slot-table entry of this thread's load j of the tile `sp` describes
  // (past the block's end it reads the next map or the padding: masked)
  auto trow = [&](const Spec& sp, int j) -> uint32_t { return stab[sp.tk0 + keyj[j]]; };
  // per-lane addresses of this thread's load j of the tile `sp` describes,
  // from its slot-table entry toff
  auto addrs = [&](const Spec& sp, Pend& pd, int j, uint32_t toff) {
    // tail slots: K of the block's first row, V out of range (zeros);
    // past the walk (nleft 0) every slot is a tail slot of row 0. The
    // validity is an opaque mask: a select on it could become a divergent
    // branch and split the fenced step.
    int m_val = -(int)(keyj[j] < sp.nleft);
    asm volatile("" : "+v"(m_val));
    const uint32_t ro = sp.base + (toff & (uint32_t)m_val);
    pd.ko[j] = min(ro, last_b) + kcst[j];   // guard: never past the last key row
    pd.vo[j] = ((ro + vcst[j]) & (uint32_t)m_val) | (kOutOfRange & ~(uint32_t)m_val);
  };
  // V copies wait one step after their K copies
  uint32_t vpend[SPW];
  auto fire_v = [&](int stage, int j) {
    const int s = wave * SPW + j;
    dma16_buf(vrsrc, vpend[j], lds_addr(vst + stage * TILE_BYTES + s * 1024));
  };
  // load j of a refill: V of tile s + AHEAD - 1 (addresses from the step
  // before) into vstage, then K of tile s + AHEAD into kstage, whose V
  // addresses replace the ones just used
  auto fire = [&](const Pend& pd, int kstage, int vstage, int j) {
    const int s = wave * SPW + j;
    fire_v(vstage, j);
    dma16(kh, pd.ko[j], lds_addr(kst + kstage * TILE_BYTES + s * 1024));
    vpend[j] = pd.vo[j];
  };
  // K of the tile `sp` describes into `stage` now, V addresses kept for
  // fire_v (the prologue)
  auto issue_k = [&](const Spec& sp, int stage) {
    Pend pd;
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      addrs(sp, pd, j, trow(sp, j));
      const int s = wave * SPW + j;
      dma16(kh, pd.ko[j], lds_addr(kst + stage * TILE_BYTES + s * 1024));
      vpend[j] = pd.vo[j];
    }
  };

  // per-lane LDS offsets of the MFMA operands
  const int kswz = lane & KSWZ;                         // (32kb + l32) & KSWZ
  const int i16 = lane & 15;
  const int vrow = 4 * g + (i16 >> 2);                  // + 32kb + 16hh (+8)
  const int vcol = 2 * ((lane >> 4) & 1) + ((i16 & 3) >> 1);  // + 4db (16-byte chunk)
  const int vhalf = (i16 & 1) * 8;
  const int vfv = (D == 128) ? 4 * (vrow & 3) : 4 * ((vrow >> 1) & 1);

  constexpr int NC = D / 16;       // 16-wide head-dim steps of S^T = K Q^T
  constexpr int NVR = 4 * NKB;     // transposed reads per 32-wide head-dim block of P.V

  // K operands of the tile in `stage`: lane holds key 32kb + l32, head-dim
  // values 16c + 8g .. +7.
  auto kread = [&](int stage, int kb, int c) -> bf16x8 {
    const unsigned char* krow = kst + stage * TILE_BYTES + (32 * kb + l32) * (CPR * 16);
    return *reinterpret_cast<const bf16x8*>(krow + (((2 * c + g) ^ kswz) * 16));
  };
  // Transposed V reads of head-dim block db: read i covers key rows
  // 8i + vrow of the tile (32kb + 16hh + 8e for i = 4kb + 2hh + e).
  auto vread = [&](int stage, int db, int i) -> u32x2 {
    const unsigned char* base = vst + stage * TILE_BYTES + vrow * (CPR * 16) + ((4 * db + vcol) ^ vfv) * 16 + vhalf;
    const i16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + 8 * i * (CPR * 16)));
    return __builtin_bit_cast(u32x2, t);
  };

  // O^T += V^T P^T for the tile in `stage`, one head-dim block of 32 at a time
  auto pv = [&](int stage, const bf16x8 (&pb)[NKB][2]) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      u32x2 vr[NVR];
#pragma unroll
      for (int i = 0; i < NVR; ++i) vr[i] = vread(stage, db, i);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const u32x4 w = {vr[4 * kb + 2 * hh][0], vr[4 * kb + 2 * hh][1], vr[4 * kb + 2 * hh + 1][0],
                           vr[4 * kb + 2 * hh + 1][1]};
          oacc[db] = E::mfma(__builtin_bit_cast(bf16x8, w), pb[kb][hh], oacc[db]);
        }
    }
  };

  // x of register r of key block kb of the QK accumulators
  auto xval = [&](const f32x16 (&sa)[NKB], int kb, int r) -> float {
    if constexpr (E::kPrescale) return sa[kb][r];
    else return fmaf(sa[kb][r], cexp, mneg);
  };
  // p = 2^x of score pair k of this lane (registers r, r+1 of key block
  // pkb), packed into the P operand pn; the pair's sum goes to ps[k % 4].
  // A lane's pairs k = 8*pkb + 4*phh + i cover keys 32*pkb + 16*phh + 8*(i/2)
  // + 4g + 2*(i%2) + {0, 1}.
  constexpr int NPAIR = NKB * 8;
  auto soft_pair = [&](int kk, const f32x16 (&sa)[NKB], bf16x8 (&pn)[NKB][2], float (&ps)[4]) {
    const int pkb = kk / 8, phh = (kk % 8) / 4, i = kk % 4, r = 8 * phh + 2 * i;
    const float e0 = __builtin_amdgcn_exp2f(xval(sa, pkb, r));
    const float e1 = __builtin_amdgcn_exp2f(xval(sa, pkb, r + 1));
    uint32_t w = E::pack2(e0, e1);
    pin(w);
    ps[kk % 4] = E::sum2(w, ps[kk % 4]);
    pin(ps[kk % 4]);
    u32x4 t = __builtin_bit_cast(u32x4, pn[pkb][phh]);
    t[i] = w;
    pn[pkb][phh] = __builtin_bit_cast(bf16x8, t);
  };

  // soft_pair in three steps, for the pipelined step: the two exponentials,
  // their packing into pn, and the pair's sum
  auto soft_exp = [&](int kk, const f32x16 (&sa)[NKB], f32x2 (&ex)[NPAIR]) {
    const int pkb = kk / 8, phh = (kk % 8) / 4, i = kk % 4, r = 8 * phh + 2 * i;
    float e0 = __builtin_amdgcn_exp2f(xval(sa, pkb, r));
    float e1 = __builtin_amdgcn_exp2f(xval(sa, pkb, r + 1));
    pin(e0);
    pin(e1);
    ex[kk] = f32x2{e0, e1};
  };
  // (pn[pkb][phh] is written whole once its four pairs are packed: the step
  // packs into the P it reads, and a chunk's old P is dead by then)
  auto soft_pack = [&](int kk, const f32x2 (&ex)[NPAIR], uint32_t (&wp)[NPAIR], bf16x8 (&pn)[NKB][2]) {
    const int pkb = kk / 8, phh = (kk % 8) / 4, i = kk % 4;
    uint32_t w = E::pack2(ex[kk][0], ex[kk][1]);
    pin(w);
    wp[kk] = w;
    if (i == 3) pn[pkb][phh] = __builtin_bit_cast(bf16x8, u32x4{wp[kk - 3], wp[kk - 2], wp[kk - 1], w});
  };
  auto soft_sum = [&](int kk, const uint32_t (&wp)[NPAIR], float (&ps)[4]) {
    ps[kk % 4] = E::sum2(wp[kk], ps[kk % 4]);
    pin(ps[kk % 4]);
  };

  // The slow path of the softmax of one tile (the first tile, or a tile
  // whose sum of p left the bound in some row): rows that need it (both
  // lanes of a row decide together) raise m to their maximum x over the
  // tile, the tile's p and sums are recomputed, and O and l of those rows
  // are rescaled by 2^-delta. Returns the tile's sum of p of this lane.
  auto raise_offset = [&](f32x16 (&sa)[NKB], bf16x8 (&pn)[NKB][2], bool need, bool first) -> float {
    float mx = xval(sa, 0, 0);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, xval(sa, kb, r));
    const f32x2 hm = halves(mx);
    const f32x2 hn = halves(need ? 1.f : 0.f);
    const bool needr = first || hn[0] + hn[1] > 0.f;
    const float delta = needr ? fmaxf(hm[0], hm[1]) : 0.f;
    if constexpr (E::kPrescale) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) sa[kb] -= delta;
      negm -= delta;
    }
    mneg -= delta;
    float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < NPAIR; ++kk) soft_pair(kk, sa, pn, ps);
    if (!first) {
      const float alpha = __builtin_amdgcn_exp2f(-delta);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
      lrow *= alpha;
    }
    return (ps[0] + ps[1]) + (ps[2] + ps[3]);
  };

  // One pipelined step, in a fixed issue order of 32 (D = 128) or 16
  // (D = 64) slots of one MFMA each, fenced so that the compiler keeps the
  // order: first the QK MFMAs of tile `ks` with the K reads KA slots ahead
  // and, in the last slots, the V operands of the first P.V slots; then the
  // P.V MFMAs of tile `vs_` (P of the previous step in pb) with their V
  // operands read VRA slots ahead and, between them, the exponentials of
  // the new scores in pairs, packed into pb as each 16-key chunk of the old
  // P is done with, and their sums. `pre` runs in the first slot, after its
  // MFMA (the walker's next tile: scalar work that the other wave's matrix
  // ops cover). WITH_PV false (the first tile) runs only the QK half; SOFT
  // false leaves the exponentials out. Tail tiles need no masking here:
  // their key slots past the block's end repeat the block's first row and
  // their V rows are zero; `tail_sum` then removes those slots from the row
  // sum.
  auto step = [&](auto with_pv, auto soft, auto pre, int ks, int vs_, bf16x8 (&pb)[NKB][2], f32x16 (&sa)[NKB],
                  float (&ps)[4], const Spec& sp, int kstage, int vstage) {
    constexpr bool WITH_PV = decltype(with_pv)::value;
    constexpr bool SOFT = decltype(soft)::value;
    constexpr int KA = 4;                   // K reads ahead of their MFMA
    constexpr int NQ = NKB * NC;            // QK MFMAs
    constexpr int NDB = D / 32;             // head-dim blocks of P.V
    constexpr int NP = NDB * 2 * NKB;       // P.V MFMAs
    constexpr int VRA = 4;                  // V operands read ahead of their MFMA
    static_assert(NPAIR % NP == 0 && VRA <= NQ, "schedule shape");
    bf16x8 kop[NQ];
    u32x4 vop[NP];
    Pend pd;
    int tv[SPW];
    f32x2 ex[NPAIR];       // exponentials of each pair, packed a slot later
    uint32_t wp[NPAIR];    // packed pairs, summed a slot later
    // V operand of P.V slot p: 16-key chunk p / NDB of head-dim block p % NDB
    auto vop_read = [&](int p) {
      const int ch = p / NDB, db = p % NDB;
      const u32x2 a0 = vread(vs_, db, 2 * ch), a1 = vread(vs_, db, 2 * ch + 1);
      vop[p] = u32x4{a0[0], a0[1], a1[0], a1[1]};
    };
    // load j: slot-table read in slot rd_slot(j), addresses and copies in
    // slot NQ/2 + fire_gap(j) (odd slots when there is room, else one load
    // per slot)
    static_assert(SPW <= NQ / 2, "one load per slot");
    constexpr bool SPREAD = 1 + 2 * (SPW - 1) < NQ / 2;
    auto rd_slot = [](int j) { return SPREAD ? 1 + 2 * j : (j * (NQ / 2)) / SPW; };
    auto fire_gap = [](int j) { return SPREAD ? 2 * j : (j * (NQ / 2)) / SPW; };
#pragma unroll
    for (int i = 0; i < KA; ++i) kop[i] = kread(ks, i / NC, i % NC);
#pragma unroll
    for (int qq = 0; qq < NQ; ++qq) {
      if (qq + KA < NQ) kop[qq + KA] = kread(ks, (qq + KA) / NC, (qq + KA) % NC);
      // the first P.V slots' V operands in the last VRA slots
      if (WITH_PV && qq >= NQ - VRA) vop_read(qq - (NQ - VRA));
      const int kb = qq / NC, c = qq % NC;
      sa[kb] = E::mfma(kop[qq], qreg[c], c != 0 ? sa[kb] : E::kPrescale ? negm : f32x16{});
      if (qq == 0) pre();
      // the refill of the stage freed by this step's barrier: slot-table
      // read of load j in slot 1 + 2j, its addresses and copies in slot
      // NQ/2 + 2j
#pragma unroll
      for (int j = 0; j < SPW; ++j) {
        if (qq == rd_slot(j)) tv[j] = trow(sp, j);
        if (qq == NQ / 2 + fire_gap(j)) {
          addrs(sp, pd, j, tv[j]);
          fire(pd, kstage, vstage, j);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // P.V with the head-dim block innermost: chunk ch of P is last read in
    // slot NDB*ch + NDB - 1, and the new P of that chunk is packed into the
    // same registers from slot NDB*(ch + 1) on.
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int ch = p / NDB, db = p % NDB;
      if constexpr (WITH_PV) {
        if (p + VRA < NP) vop_read(p + VRA);
        oacc[db] = E::mfma(__builtin_bit_cast(bf16x8, vop[p]), pb[ch / 2][ch % 2], oacc[db]);
      }
      if constexpr (SOFT) {
        // exponentials of this slot's pairs, packing of the previous slot's,
        // sums of the slot before: no result is used in the slot that makes it
#pragma unroll
        for (int kk = p * (NPAIR / NP); kk < (p + 1) * (NPAIR / NP); ++kk) soft_exp(kk, sa, ex);
        if (p >= 1) {
#pragma unroll
          for (int kk = (p - 1) * (NPAIR / NP); kk < p * (NPAIR / NP); ++kk) soft_pack(kk, ex, wp, pb);
        }
        if (p >= 2) {
#pragma unroll
          for (int kk = (p - 2) * (NPAIR / NP); kk < (p - 1) * (NPAIR / NP); ++kk) soft_sum(kk, wp, ps);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (SOFT) {   // the last two slots' packing and sums
#pragma unroll
      for (int kk = (NP - 1) * (NPAIR / NP); kk < NPAIR; ++kk) soft_pack(kk, ex, wp, pb);
#pragma unroll
      for (int kk = (NP - 2) * (NPAIR / NP); kk < NPAIR; ++kk) soft_sum(kk, wp, ps);
    }
  };

  // Row-sum correction of a tail tile: a lane's slots past the block's end
  // all hold the score of the block's first row, so they added the same p
  // to the row sum; `plast` is p of the lane's last slot (key
  // 32(NKB-1) + 24 + 4g + 3), always among them when the lane has any.
  auto tail_sum = [&](uint64_t cmask, float plast) {
    const uint64_t mine = g ? 0xF0F0F0F0F0F0F0F0ull : 0x0F0F0F0F0F0F0F0Full;
    const int ninv = __builtin_popcountll(~cmask & FULLM & mine);
    lrow = fmaf(-(float)ninv, plast, lrow);
  };
  // p of the lane's last slot, as the row sum added it
  auto last_p = [&](const bf16x8 (&pn)[NKB][2]) -> float {
    return E::hi(__builtin_bit_cast(u32x4, pn[NKB - 1][1])[3]);
  };

  // Publish: every wave has waited for its own loads of the tiles needed
  // next. A plain s_barrier suffices; __syncthreads would also wait for the
  // tiles still in flight.
  auto barrier = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // Tile ring: slot i holds the i-th tile from the one the next step starts
  // with. AHEAD tiles are in flight when a step begins.
  constexpr int AHEAD = NSTAGE - BSTEP;
  static_assert(BSTEP == 1 || (BSTEP == 2 && NSTAGE % 2 == 0 && AHEAD >= 2), "barrier spacing");
  uint64_t mring[AHEAD + 1];
  bool ering[AHEAD + 1];
#pragma unroll
  for (int i = 0; i <= AHEAD; ++i) {
    ering[i] = false;
    mring[i] = 0;
  }
  // prologue: K of tiles 0 .. AHEAD-1 and V of tiles 0 .. AHEAD-2, in the
  // order the steps would issue them
#pragma unroll
  for (int i = 0; i < AHEAD; ++i) {
    if (i > 0 && ering[i - 1]) {
#pragma unroll
      for (int j = 0; j < SPW; ++j) fire_v(i - 1, j);
    }
    if (ibi < nkept) {
      Spec sp0;
      spec(sp0, mring[i], ering[i]);
      issue_k(sp0, i);
    }
  }
  // wait for this wave's copies of the K of ring slot 0 and of the V of the
  // tile before it (both issued in the same step; later ones may stay in
  // flight)
  auto wait_first = [&]() {
    if constexpr (AHEAD >= 3) {
      if (ering[2]) wait_vmcnt<2 * VM_PER_TILE>();
      else if (ering[1]) wait_vmcnt<VM_PER_TILE>();
      else wait_vmcnt<0>();
    } else if constexpr (AHEAD == 2) {
      if (ering[1]) wait_vmcnt<VM_PER_TILE>(); else wait_vmcnt<0>();
    } else {
      wait_vmcnt<0>();
    }
  };
  auto shift = [&]() {
#pragma unroll
    for (int i = 0; i < AHEAD; ++i) {
      mring[i] = mring[i + 1];
      ering[i] = ering[i + 1];
    }
  };

  using T_ = std::true_type;
  using F_ = std::false_type;
  // The tile loop, once for waves with query rows (ACTIVE) and once for
  // waves without (they only load their share of the tiles and keep the
  // barriers); two loops instead of a branch inside one keep the O
  // accumulators in fixed registers.
  auto run = [&](auto active) {
    constexpr bool ACTIVE = decltype(active)::value;
    // Software pipeline. Tile t sits in stage t % NSTAGE. Step j runs QK
    // of tile j and the P.V of tile j-1 (whose P the previous step made),
    // with the exponentials of tile j on the vector ALUs while the P.V
    // matrix ops run. The barrier before every BSTEP-th step publishes what
    // the next BSTEP steps read; every wave has then finished the steps
    // before it, so the stages they read are free, and step j copies K of
    // tile j + AHEAD and V of tile j + AHEAD - 1 into them.
    bf16x8 pb[NKB][2];
    Spec sp;
    auto fire_all = [&](int kstage, int vstage) {
      Pend pd;
      int tv[SPW];
#pragma unroll
      for (int j = 0; j < SPW; ++j) tv[j] = trow(sp, j);
#pragma unroll
      for (int j = 0; j < SPW; ++j) {
        addrs(sp, pd, j, tv[j]);
        fire(pd, kstage, vstage, j);
      }
    };
    // first tile: QK, then the offset from its row maximum (every kept list
    // has a tile)
    spec(sp, mring[AHEAD], ering[AHEAD]);
    if constexpr (BSTEP == 1) wait_first(); else wait_vmcnt<0>();
    barrier();
    if constexpr (ACTIVE) {
      f32x16 sa[NKB];
      float ps[4];
      step(F_{}, F_{}, [] {}, 0, 0, pb, sa, ps, sp, AHEAD, AHEAD - 1);
      lrow = raise_offset(sa, pb, true, true);
      if (mring[0] != FULLM) tail_sum(mring[0], last_p(pb));
    } else {
      fire_all(AHEAD, AHEAD - 1);
    }
    shift();
    int cur = 1, prev = 0;
    // steady state; the step after the last tile runs the last P.V only
#pragma unroll 1
    while (true) {
      const bool have = ering[0];
      const int fst = cur + AHEAD >= NSTAGE ? cur + AHEAD - NSTAGE : cur + AHEAD;   // K refill
      const int vfst = fst == 0 ? NSTAGE - 1 : fst - 1;                               // V refill
      if (!ACTIVE && have) spec(sp, mring[AHEAD], ering[AHEAD]);
      // the last P.V reads V of the last tile, copied one step after its K
      if constexpr (BSTEP == 1) {
        if (have) wait_first(); else wait_vmcnt<0>();
        barrier();
      } else if ((cur & 1) == 0 || !have) {  // every other step, and before the last P.V
        wait_vmcnt<0>();
        barrier();
      }
      if (!have) {
        if constexpr (ACTIVE) pv(prev, pb);
        break;
      }
      if constexpr (ACTIVE) {
        f32x16 sa[NKB];
        float ps[4] = {0.f, 0.f, 0.f, 0.f};
        step(T_{}, T_{}, [&] { spec(sp, mring[AHEAD], ering[AHEAD]); }, cur, prev, pb, sa, ps, sp, fst, vfst);
        const float psum = (ps[0] + ps[1]) + (ps[2] + ps[3]);
        const bool need = !(psum <= E::kSumLimit);   // NaN or inf included
        if (__ballot(need) != 0) lrow += raise_offset(sa, pb, need, false);
        else lrow += psum;
        if (mring[0] != FULLM) tail_sum(mring[0], last_p(pb));
      } else {
        fire_all(fst, vfst);
      }
      prev = cur;
      cur = cur + 1 == NSTAGE ? 0 : cur + 1;
      shift();
    }
  };
  if (!wave_active) {
    run(F_{});
    return;
  }
  run(T_{});

  // ---- normalise and store in raster order
  const f32x2 hl = halves(lrow);
  const float inv = 1.f / (hl[0] + hl[1]);
  if (qrow >= 0) {
    __bf16* dst = oh + (int64_t)qrow * a.osn + 4 * g;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        u32x2 w;
        w[0] = E::pack2(oacc[db][4 * r4] * inv, oacc[db][4 * r4 + 1] * inv);
        w[1] = E::pack2(oacc[db][4 * r4 + 2] * inv, oacc[db][4 * r4 + 3] * inv);
        *reinterpret_cast<u32x2*>(dst + 32 * db + 8 * r4) = w;
      }
  }
}

// Workgroups of `func` resident at once on one XCD (8 per gfx950 device):
// the occupancy per CU times the CUs of an XCD. Cached per device and LDS
// size; -1 if a query fails.
int resident_per_xcd(const void* func, int threads, size_t lds) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  // one atomic word per slot: a 48-bit key (never 0) over a 16-bit value
  static std::atomic<uint64_t> cache[8];
  uint64_t h = (uint64_t)(uintptr_t)func * 0x9E3779B97F4A7C15ull;
  h ^= ((uint64_t)lds << 17) ^ ((uint64_t)threads << 3) ^ ((uint64_t)(uint32_t)dev << 40);
  const uint64_t key = ((h >> 16) & 0xFFFFFFFFFFFFull) | 1ull;
  std::atomic<uint64_t>& slot = cache[key % 8];
  const uint64_t w = slot.load(std::memory_order_relaxed);
  if ((w >> 16) == key) return (int)(w & 0xFFFFu);
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, func, threads, lds) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  const int conc = per_cu * (cus / 8);
  if (conc < 0 || conc > 0xFFFF) return -1;
  slot.store((key << 16) | (uint64_t)conc, std::memory_order_relaxed);
  return conc;
}

// LDS bytes of one launch: K and V stages, the slot tables and the
// kept-block table.
template <int D, int NSTAGE, int KT>
size_t attend_lds_bytes(const VsaArgs& a) {
  return (size_t)2 * NSTAGE * KT * D * 2 + slot_table_bytes(a.gk.V, KT) + (size_t)(a.gk.Pb + a.topk) * 8;
}

template <int D, int NW, int NSTAGE, int KT, int WPE, bool F16, int BSTEP>
hipError_t launch(const VsaArgs& a, const void* q, const void* k, const void* v, const int32_t* sel, void* o,
                  hipStream_t stream) {
  const size_t lds = attend_lds_bytes<D, NSTAGE, KT>(a);
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  if (lds > 65536) {
    static std::atomic<uint64_t> raised{0};
    const hipError_t e = vsa_raise_lds_limit(
        reinterpret_cast<const void*>(&vsa_attend_kernel<D, NW, NSTAGE, KT, WPE, F16, BSTEP>), raised);
    if (e != hipSuccess) return e;
  }
  VsaArgs b = a;
  constexpr int RW = NW * 32;  // query slots per workgroup
  b.tiles = (a.gq.V + RW - 1) / RW;
  const int64_t nunits = (int64_t)a.B * a.Hh * a.nq * b.tiles;
  if (nunits > (int64_t)INT32_MAX / 2 - 64) return hipErrorInvalidValue;
  const int conc = resident_per_xcd(
      reinterpret_cast<const void*>(&vsa_attend_kernel<D, NW, NSTAGE, KT, WPE, F16, BSTEP>), NW * 64, lds);
  if (conc <= 0) return hipErrorInvalidValue;
  // Small-cube kernel: stagger the walks over 5/4 of the resident set. The
  // period of start positions is a tuning choice: measured against 1x to 3x
  // the resident count on both 64-token-cube workloads, 1.2x to 1.25x was
  // best (3% less time than 1x on 960 cubes).
  b.walk_conc = NW == 2 ? conc + conc / 4 : 0;
  // Large-cube kernel: when the last round of workgroups on each XCD is at
  // most half full, its units run as half-row workgroups (twice as many,
  // each quicker: one wave per SIMD instead of two).
  const int64_t per_xcd = (nunits + 7) / 8;
  const int64_t rem = per_xcd % conc;
  b.split_tail = (NW == 8 && rem > 0 && 2 * rem <= conc) ? (int32_t)rem : 0;
  dim3 grid((unsigned)(8 * (per_xcd + b.split_tail)));
  hipLaunchKernelGGL((vsa_attend_kernel<D, NW, NSTAGE, KT, WPE, F16, BSTEP>), grid, dim3(NW * 64), lds, stream, b,
                     (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, sel, (__bf16*)o);
  return hipGetLastError();
}

}  // namespace

// Tilings, all on the pipelined step: cubes of up to 64 tokens use 2-wave
// workgroups (64 query rows) with 32-key tiles in rings of two (32 KB of
// K/V stages for D = 128, so four workgroups share a CU) and a barrier per
// tile; larger cubes use 8-wave workgroups (256 query rows) with 64-key
// tiles, for D = 128 in rings of four with one barrier per two tiles
// (128 KB), or in rings of two with a barrier per tile when the slot and
// kept-block tables leave no room for four; for D = 64 in rings of three
// with a barrier per tile.
template <bool F16>
static hipError_t dispatch(const VsaArgs& a, int variant, const void* q, const void* k, const void* v,
                           const int32_t* sel, void* o, hipStream_t stream) {
  if (a.D == 128) {
    if (variant == VSA_ATTEND_ROWS64) return launch<128, 2, 2, 32, 2, F16, 1>(a, q, k, v, sel, o, stream);
    if (attend_lds_bytes<128, 4, 64>(a) <= 160 * 1024) return launch<128, 8, 4, 64, 2, F16, 2>(a, q, k, v, sel, o, stream);
    return launch<128, 8, 2, 64, 2, F16, 1>(a, q, k, v, sel, o, stream);
  }
  if (variant == VSA_ATTEND_ROWS64) return launch<64, 2, 2, 32, 2, F16, 1>(a, q, k, v, sel, o, stream);
  return launch<64, 8, 3, 64, 2, F16, 1>(a, q, k, v, sel, o, stream);
}

hipError_t vsa_launch_attend(const VsaArgs& a, int variant, const void* q, const void* k, const void* v,
                             const int32_t* sel, void* o, hipStream_t stream) {
  return a.f16 ? dispatch<true>(a, variant, q, k, v, sel, o, stream)
               : dispatch<false>(a, variant, q, k, v, sel, o, stream);
}
