// Device-side types and the raster <-> block index map shared by the
// block-sparse attention kernels (gfx950, wave64).
//
// Index map (fastbsa package page, section "How it works": the raster to
// block-contiguous map is evaluated inside the kernels, so q, k and v are
// never permuted through HBM). A block's tokens are addressed by a compact
// slot r in 0..n-1, where n is the number of valid tokens: for a video cube
// with valid extents (et, eh, ew) slot r is (tt, hh, ww) in raster order
// inside the cube, token row P + ((t0+tt)*H + h0+hh)*W + w0+ww; for prefix
// block p slot r is token row p*V + r. Partial edge cubes therefore have no
// holes: only the last 64-token tile of a block can be short.
#ifndef VSA_DEVICE_H
#define VSA_DEVICE_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

// Host: raises a kernel's dynamic LDS limit to the 160 KB of a gfx950 CU,
// once per device (the attribute belongs to each device's copy of the
// kernel). `done` holds one bit per device id below 64; for larger ids the
// attribute is set on every call.
inline hipError_t vsa_raise_lds_limit(const void* func, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev >= 0 && dev < 64 ? (1ull << dev) : 0ull;
  if (bit != 0 && (done.load(std::memory_order_acquire) & bit) != 0) return hipSuccess;
  e = hipFuncSetAttribute(func, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (e == hipSuccess && bit != 0) done.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// One side's grid and its cutting into blocks: q's (query blocks) or
// k/v's (key blocks). The two differ when q and k/v lie on different
// latent grids or use different cube shapes (fastbsa package page, section
// "Use": separate latent and chunk shapes for q and k).
struct VsaGrid {
  int32_t T, H, W;
  int32_t ct, ch, cw;
  int32_t nT, nH, nW;
  int32_t P, V, Pb, nb;  // prefix tokens, cube volume, prefix blocks, cubes
  uint64_t magic_nW;     // ceil(2^32 / nW): floor(x / nW) = (x * magic) >> 32 for x < 2^16
  uint64_t magic_nH;     // ceil(2^32 / nH)
  // Division magics of the valid extents of cubes: ew in {cw, W - (nW-1)*cw}
  // (index 0: whole, 1: tail) and eh*ew with index 2*[eh is the tail] +
  // [ew is the tail].
  uint64_t magic_ew[2];
  uint64_t magic_ehw[4];
};

// Everything the kernels need, passed by value.
struct VsaArgs {
  int32_t B, Hh, D;
  VsaGrid gq, gk;        // query side, key/value side
  int32_t nq;            // query blocks: gq.Pb + gq.nb
  int32_t nb;            // key cubes: gk.nb (the ids sel holds)
  int32_t topk;
  int64_t sb, sh;        // q batch and head strides (elements)
  int32_t sn;            // q token stride (elements)
  int64_t ksb, ksh;      // k and v strides
  int32_t ksn;
  int64_t osb, osh;
  int32_t osn;
  float scale_log2e;     // head_dim^-1/2 * log2(e)
  int32_t select_rows;   // query blocks per score/top-k workgroup
  int32_t tiles;         // query row tiles per query block
  int32_t f16;           // q, k, v, o are fp16 (else bf16)
  int32_t walk_conc;     // attention: period, in dispatch order within an
                         // XCD, of the walks' staggered start positions
                         // (about the resident workgroups; 0: no stagger)
  int32_t split_tail;    // attention: units at the end of each XCD's range
                         // that run as two half-row workgroups (0: none)
};

// Valid region of one block: first token row, extents of the (tt, hh, ww)
// box (prefix blocks use (1, 1, n)) and valid token count.
struct BlockExt {
  int32_t base;
  int32_t eh, ew;
  int32_t n;
};

__device__ __forceinline__ BlockExt block_ext(const VsaGrid& g, int32_t blk) {
  BlockExt e;
  if (blk < g.Pb) {
    const int32_t s = blk * g.V;
    const int32_t n = min(g.V, g.P - s);
    e.base = s;
    e.eh = 1;
    e.ew = n;
    e.n = n;
    return e;
  }
  const int32_t c = blk - g.Pb;
  const int32_t bw = c % g.nW;
  const int32_t rest = c / g.nW;
  const int32_t bh = rest % g.nH;
  const int32_t bt = rest / g.nH;
  const int32_t t0 = bt * g.ct, h0 = bh * g.ch, w0 = bw * g.cw;
  const int32_t et = min(g.ct, g.T - t0);
  e.eh = min(g.ch, g.H - h0);
  e.ew = min(g.cw, g.W - w0);
  e.base = g.P + (t0 * g.H + h0) * g.W + w0;
  e.n = et * e.eh * e.ew;
  return e;
}

// Token row of compact slot r (0 <= r < e.n) of a block.
__device__ __forceinline__ int32_t slot_row(const VsaGrid& g, const BlockExt& e, int32_t r) {
  const uint32_t ehw = (uint32_t)(e.eh * e.ew);
  const uint32_t tt = (uint32_t)r / ehw;
  const uint32_t rem = (uint32_t)r - tt * ehw;
  const uint32_t hh = rem / (uint32_t)e.ew;
  const uint32_t ww = rem - hh * (uint32_t)e.ew;
  return e.base + ((int32_t)tt * g.H + (int32_t)hh) * g.W + (int32_t)ww;
}

__device__ __forceinline__ uint32_t orderable_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

#endif
