// Block-sparse flash attention over the kept blocks ("FastVideo VSA" user
// guide, opening definition: attention only against the selected top-k
// blocks; section "Choose top-k": prefix blocks are always kept; section
// "Verify routing and fallback": non-causal, scale head_size^-1/2).
//
// Work split. One workgroup owns RW = NW*32*QB query slots of one query block
// of one (batch, head); each wave owns 32*QB of them. The kept key blocks
// (all prefix blocks, then the selected cubes in ascending order) are walked
// in tiles of 64 key slots.
//
// Index map (fastbsa package page, section "How it works": the raster to
// block map is evaluated inside the kernel). A block's V = ct*ch*cw slots are
// numbered s = (tt*ch + hh)*cw + ww. At start-up the workgroup tabulates,
// for every slot, its row offset (tt*H + hh)*W + ww from the cube's first
// token and its packed (tt, hh, ww); afterwards a slot's token row is one LDS
// read plus an add, with no division. A slot is valid when (tt, hh, ww) lies
// inside the block's valid extents (partial cubes at the far edge of an axis);
// prefix block slots are the rows p*V + s, valid below the prefix length.
// Invalid key slots load as zero and are masked to -inf, so only tiles of
// partial blocks pay for masking; a block's tiles stop at its last valid slot.
//
// Pipeline. K and V^T tiles are double-buffered in LDS. While tile i is
// computed from one buffer, tile i+1's global loads are in flight into
// registers; they are written to the other buffer after the math, followed by
// the tile's only barrier.
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
// The 8 keys a lane feeds to one P.V step are {4g..4g+3, 8+4g..8+4g+3} of a
// 16-key group, so V^T is stored with each 16-key group permuted as
// (0-3, 8-11, 4-7, 12-15); one 16-byte LDS read then yields the matching V
// operand. Every lane owns one query row: the row max and sum need one
// exchange between the two lane halves and rescaling O is a per-lane scalar.
// Softmax runs in base 2 on unscaled scores: p = 2^(s*c - m*c) with
// c = head_dim^-1/2 * log2(e), the same softmax.

#include "vsa_device.h"
#include "vsa_limits.h"

namespace {

constexpr int KT = 64;  // key slots per tile

__device__ __forceinline__ uint32_t pack_bf16x2(float x, float y) {
  const __bf16 a = (__bf16)x, b = (__bf16)y;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// Packed slot coordinates: tt | hh << 10 | ww << 20 (each < 1024).
__device__ __forceinline__ bool slot_valid(uint32_t crd, uint32_t ext) {
  return ((crd & 1023u) < (ext & 1023u)) & (((crd >> 10) & 1023u) < ((ext >> 10) & 1023u)) &
         ((crd >> 20) < (ext >> 20));
}

// Valid region of a kept or query block in slot space.
struct Blk {
  int32_t base;     // first token row
  uint32_t ext;     // packed valid extents (et, eh, ew); prefix blocks (1, 1, n)
  int32_t ntiles;   // 64-slot tiles up to the last valid slot
  bool prefix;
  bool full;        // every slot below V valid
};

__device__ __forceinline__ Blk describe_block(const VsaArgs& a, int32_t blk) {
  Blk d;
  if (blk < a.Pb) {
    const int32_t s = blk * a.V;
    const int32_t n = min(a.V, a.P - s);
    d.base = s;
    d.ext = 1u | (1u << 10) | ((uint32_t)n << 20);
    d.ntiles = (n + KT - 1) / KT;
    d.prefix = true;
    d.full = n == a.V;
    return d;
  }
  const int32_t c = blk - a.Pb;
  const int32_t bw = c % a.nW;
  const int32_t rest = c / a.nW;
  const int32_t bh = rest % a.nH;
  const int32_t bt = rest / a.nH;
  const int32_t t0 = bt * a.ct, h0 = bh * a.ch, w0 = bw * a.cw;
  const int32_t et = min(a.ct, a.T - t0), eh = min(a.ch, a.H - h0), ew = min(a.cw, a.W - w0);
  d.base = a.P + (t0 * a.H + h0) * a.W + w0;
  d.ext = (uint32_t)et | ((uint32_t)eh << 10) | ((uint32_t)ew << 20);
  const int32_t last = ((et - 1) * a.ch + (eh - 1)) * a.cw + (ew - 1);
  d.ntiles = last / KT + 1;
  d.prefix = false;
  d.full = (et == a.ct) & (eh == a.ch) & (ew == a.cw);
  return d;
}

template <int D, int NW, int QB, int VCAP>
__global__ __launch_bounds__(NW * 64) void vsa_attend_kernel(VsaArgs a, const __bf16* __restrict__ q,
                                                             const __bf16* __restrict__ k,
                                                             const __bf16* __restrict__ v,
                                                             const int32_t* __restrict__ sel,
                                                             __bf16* __restrict__ o) {
  constexpr int NT = NW * 64;
  constexpr int CPR = D / 8;               // 16-byte chunks per key row
  constexpr int RW = NW * 32 * QB;         // query slots per workgroup
  constexpr int KCH = KT * CPR / NT;       // K chunks per thread per tile
  constexpr int VTASKS = (KT / 2) * CPR;   // (key pair, 8 head-dim) tasks
  constexpr int VPT = (VTASKS + NT - 1) / NT;  // V tasks per thread per tile
  constexpr int KSWZ = (CPR < 16 ? CPR : 16) - 1;  // K chunk swizzle mask
  static_assert(KT * CPR % NT == 0, "K tile must split evenly");

  __shared__ __align__(16) __bf16 Ks[2][KT * D];
  __shared__ __align__(16) __bf16 Vt[2][D * KT];
  __shared__ int32_t srel[VCAP];
  __shared__ uint32_t scrd[VCAP];

  int bid = blockIdx.x;
  const int tile = bid % a.tiles;
  bid /= a.tiles;
  const int qblk = bid % a.nq;
  const int bh = bid / a.nq;
  const int b = bh / a.Hh, h = bh - b * a.Hh;
  const Blk qd = describe_block(a, qblk);
  const int slot0 = tile * RW;
  if (slot0 >= qd.ntiles * KT) return;

  const int tid = threadIdx.x;
  for (int s = tid; s < a.V; s += NT) {
    const int chw = a.ch * a.cw;
    const int tt = s / chw;
    const int rem = s - tt * chw;
    const int hh = rem / a.cw;
    const int ww = rem - hh * a.cw;
    srel[s] = (tt * a.H + hh) * a.W + ww;
    scrd[s] = (uint32_t)tt | ((uint32_t)hh << 10) | ((uint32_t)ww << 20);
  }
  __syncthreads();

  const int64_t in_off = (int64_t)b * a.sb + (int64_t)h * a.sh;
  const __bf16* qh = q + in_off;
  const __bf16* kh = k + in_off;
  const __bf16* vh = v + in_off;
  __bf16* oh = o + (int64_t)b * a.osb + (int64_t)h * a.osh;
  const int32_t* selrow = sel + ((int64_t)bh * a.nq + qblk) * a.topk;

  const int wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, g = lane >> 5;

  // token row of slot s of block d, or -1 when the slot is not valid
  auto slot_row = [&](const Blk& d, int s) -> int {
    if (s >= a.V) return -1;
    const uint32_t crd = d.prefix ? ((uint32_t)s << 20) : scrd[s];
    if (!slot_valid(crd, d.ext)) return -1;
    return d.base + (d.prefix ? s : srel[s]);
  };

  // ---- Q rows of this wave, in MFMA B-operand layout
  int qrow[QB];
  bf16x8 qreg[QB][D / 16];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    qrow[qb] = slot_row(qd, slot0 + wave * 32 * QB + qb * 32 + l32);
    if (qrow[qb] >= 0) {
      const __bf16* src = qh + (int64_t)qrow[qb] * a.sn + 8 * g;
#pragma unroll
      for (int c = 0; c < D / 16; ++c) qreg[qb][c] = *reinterpret_cast<const bf16x8*>(src + 16 * c);
    } else {
#pragma unroll
      for (int c = 0; c < D / 16; ++c) qreg[qb][c] = bf16x8{};
    }
  }
  bool wave_active = false;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) wave_active |= qrow[qb] >= 0;
  wave_active = __ballot(wave_active) != 0;

  f32x16 oacc[QB][D / 32];
  float mrow[QB], lrow[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    mrow[qb] = -INFINITY;
    lrow[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[qb][db] = f32x16{};
  }

  // ---- kept-block walk
  const int nkept = a.Pb + a.topk;
  auto kept_block = [&](int i) -> int {
    if (i < a.Pb) return i;
    int c = selrow[i - a.Pb];
    c = c < 0 ? 0 : (c >= a.nb ? a.nb - 1 : c);
    return a.Pb + c;
  };

  u32x4 kbuf[KCH];
  u32x4 vbuf[VPT][2];

  auto load_tile = [&](const Blk& d, int t) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int idx = tid + i * NT;
      const int key = idx / CPR, c = idx % CPR;
      const int row = slot_row(d, t * KT + key);
      kbuf[i] = row >= 0 ? *reinterpret_cast<const u32x4*>(kh + (int64_t)row * a.sn + c * 8) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int task = tid + i * NT;
      const int kp = task % (KT / 2), e8 = task / (KT / 2);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = task < VTASKS ? slot_row(d, t * KT + 2 * kp + j) : -1;
        vbuf[i][j] = row >= 0 ? *reinterpret_cast<const u32x4*>(vh + (int64_t)row * a.sn + e8 * 8)
                              : u32x4{0, 0, 0, 0};
      }
    }
  };

  auto store_tile = [&](int buf) {
    __bf16* ks = Ks[buf];
    __bf16* vt = Vt[buf];
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int idx = tid + i * NT;
      const int key = idx / CPR, c = idx % CPR;
      *reinterpret_cast<u32x4*>(ks + key * D + ((c ^ (key & KSWZ)) * 8)) = kbuf[i];
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int task = tid + i * NT;
      if (task >= VTASKS) break;
      const int kp = task % (KT / 2), e8 = task / (KT / 2);
      // keys 2kp, 2kp+1 -> positions inside the permuted 16-key group
      const int key = 2 * kp;
      const int p = (key & ~15) | (key & 3) | ((key & 4) << 1) | ((key & 8) >> 1);
      const int pc = p >> 3, off = p & 7;
#pragma unroll
      for (int ii = 0; ii < 8; ++ii) {
        const int d = 8 * e8 + ii;
        const uint32_t s = (ii & 1) ? 0x07060302u : 0x05040100u;
        const uint32_t w = __builtin_amdgcn_perm(vbuf[i][1][ii >> 1], vbuf[i][0][ii >> 1], s);
        const int swz = (d ^ (d >> 3)) & 7;
        *reinterpret_cast<uint32_t*>(vt + d * KT + ((pc ^ swz) * 8) + off) = w;
      }
    }
  };

  // tile validity bits (bit i: slot t*64 + i is valid), uniform
  auto tile_mask = [&](const Blk& d, int t) -> uint64_t {
    if (d.full && (t + 1) * KT <= a.V) return ~0ull;
    return __ballot(slot_row(d, t * KT + lane) >= 0);
  };

  const float cexp = a.scale_log2e;
  int bi = 0, kt = 0;
  Blk kd = describe_block(a, kept_block(0));
  load_tile(kd, 0);
  store_tile(0);
  uint64_t vmask = tile_mask(kd, 0);
  __syncthreads();

  int cur = 0;
#pragma unroll 1
  while (true) {
    // advance to the next tile and start its loads
    const uint64_t cmask = vmask;
    ++kt;
    if (kt >= kd.ntiles) {
      kt = 0;
      ++bi;
      if (bi < nkept) kd = describe_block(a, kept_block(bi));
    }
    const bool more = bi < nkept;
    if (more) {
      load_tile(kd, kt);
      vmask = tile_mask(kd, kt);
    }

    if (wave_active) {
      const __bf16* ks = Ks[cur];
      const __bf16* vt = Vt[cur];
      f32x16 s[QB][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[qb][kb] = f32x16{};
        const int key = 32 * kb + l32;
#pragma unroll
        for (int c = 0; c < D / 16; ++c) {
          const int chunk = 2 * c + g;
          const bf16x8 kop = *reinterpret_cast<const bf16x8*>(ks + key * D + ((chunk ^ (key & KSWZ)) * 8));
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            s[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qreg[qb][c], s[qb][kb], 0, 0, 0);
        }
      }
      if (cmask != ~0ull) {
        const uint64_t mg = cmask >> (4 * g);
        const uint32_t m0 = (uint32_t)mg, m1 = (uint32_t)(mg >> 32);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int bit = 8 * (r >> 2) + (r & 3);
          const bool v0 = (m0 >> bit) & 1u, v1 = (m1 >> bit) & 1u;
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            s[qb][0][r] = v0 ? s[qb][0][r] : -INFINITY;
            s[qb][1][r] = v1 ? s[qb][1][r] : -INFINITY;
          }
        }
      }
      bf16x8 pb[QB][2][2];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float mx = s[qb][0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[qb][kb][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float mnew = fmaxf(mrow[qb], mx);
        const float alpha = __builtin_amdgcn_exp2f((mrow[qb] - mnew) * cexp);
        const float mc = mnew * cexp;
        float psum = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = __builtin_amdgcn_exp2f(fmaf(s[qb][kb][r], cexp, -mc));
            s[qb][kb][r] = p;
            psum += p;
          }
        lrow[qb] = lrow[qb] * alpha + psum;
        mrow[qb] = mnew;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) oacc[qb][db] *= alpha;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            u32x4 w;
#pragma unroll
            for (int i = 0; i < 4; ++i)
              w[i] = pack_bf16x2(s[qb][kb][8 * hh + 2 * i], s[qb][kb][8 * hh + 2 * i + 1]);
            pb[qb][kb][hh] = __builtin_bit_cast(bf16x8, w);
          }
      }
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int d = 32 * db + l32;
        const int swz = (d ^ (d >> 3)) & 7;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int pc = 4 * kb + 2 * hh + g;
            const bf16x8 vop = *reinterpret_cast<const bf16x8*>(vt + d * KT + ((pc ^ swz) * 8));
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
              oacc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pb[qb][kb][hh], oacc[qb][db], 0, 0, 0);
          }
      }
    }
    if (!more) break;
    store_tile(cur ^ 1);
    __syncthreads();
    cur ^= 1;
  }

  // ---- normalise and store in raster order
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float ltot = lrow[qb] + __shfl_xor(lrow[qb], 32, 64);
    const float inv = 1.f / ltot;
    if (qrow[qb] >= 0) {
      __bf16* dst = oh + (int64_t)qrow[qb] * a.osn + 4 * g;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          u32x2 w;
          w[0] = pack_bf16x2(oacc[qb][db][4 * r4] * inv, oacc[qb][db][4 * r4 + 1] * inv);
          w[1] = pack_bf16x2(oacc[qb][db][4 * r4 + 2] * inv, oacc[qb][db][4 * r4 + 3] * inv);
          *reinterpret_cast<u32x2*>(dst + 32 * db + 8 * r4) = w;
        }
    }
  }
}

template <int D, int NW, int QB, int VCAP>
hipError_t launch(const VsaArgs& a, const void* q, const void* k, const void* v, const int32_t* sel, void* o,
                  hipStream_t stream) {
  dim3 grid((int64_t)a.B * a.Hh * a.nq * a.tiles);
  hipLaunchKernelGGL((vsa_attend_kernel<D, NW, QB, VCAP>), grid, dim3(NW * 64), 0, stream, a,
                     (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, sel, (__bf16*)o);
  return hipGetLastError();
}

}  // namespace

hipError_t vsa_launch_attend(const VsaArgs& a, int variant, const void* q, const void* k, const void* v,
                             const int32_t* sel, void* o, hipStream_t stream) {
  if (a.D == 128) {
    if (variant == VSA_ATTEND_ROWS64) return launch<128, 2, 1, 64>(a, q, k, v, sel, o, stream);
    return launch<128, 8, 1, VSA_MAX_CUBE_VOLUME>(a, q, k, v, sel, o, stream);
  }
  if (variant == VSA_ATTEND_ROWS64) return launch<64, 2, 1, 64>(a, q, k, v, sel, o, stream);
  return launch<64, 8, 1, VSA_MAX_CUBE_VOLUME>(a, q, k, v, sel, o, stream);
}
