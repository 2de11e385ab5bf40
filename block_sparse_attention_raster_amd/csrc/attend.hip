// Block-sparse flash attention over the kept blocks ("FastVideo VSA" user
// guide, opening definition: attention only against the selected top-k
// blocks; section "Choose top-k": prefix blocks are always kept; section
// "Verify routing and fallback": non-causal, scale head_size^-1/2).
//
// One workgroup owns up to RW = NW*32*QB query rows (compact slots) of one
// query block of one (batch, head); each wave owns 32*QB rows. The kept key
// blocks (all prefix blocks, then the selected cubes in ascending order) are
// walked in tiles of 64 compact key slots; only a block's last tile can be
// short and its missing keys are masked to -inf. Each tile is staged in LDS
// through the in-kernel index map (fastbsa package page, section "How it
// works"), with the next tile's global loads issued before the current
// tile's math.
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
// 16-key group, so V^T is stored in LDS with each 16-key group permuted as
// (0-3, 8-11, 4-7, 12-15); one 16-byte LDS read then yields the matching V
// operand. Every lane thus owns one query row: the row max and sum need one
// cross-half exchange, and the rescale of O is a per-lane scalar.
// Softmax is computed in base 2 on unscaled scores: p = 2^(s*c - m*c) with
// c = head_dim^-1/2 * log2(e), which is the same softmax.

#include "vsa_device.h"
#include "vsa_limits.h"

namespace {

constexpr int KT = 64;  // key slots per tile

__device__ __forceinline__ uint32_t perm_b32(uint32_t hi_src, uint32_t lo_src, uint32_t sel) {
  return __builtin_amdgcn_perm(hi_src, lo_src, sel);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float x, float y) {
  const __bf16 a = (__bf16)x, b = (__bf16)y;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

template <int D, int NW, int QB>
__global__ __launch_bounds__(NW * 64) void vsa_attend_kernel(VsaArgs a, const __bf16* __restrict__ q,
                                                             const __bf16* __restrict__ k,
                                                             const __bf16* __restrict__ v,
                                                             const int32_t* __restrict__ sel,
                                                             __bf16* __restrict__ o) {
  constexpr int NT = NW * 64;
  constexpr int CPR = D / 8;               // 16-byte chunks per key row
  constexpr int RW = NW * 32 * QB;         // query rows per workgroup
  constexpr int KCH = KT * CPR / NT;       // K chunks per thread per tile
  constexpr int VTASKS = (KT / 4) * CPR;   // (4 keys x 8 dims) transpose tasks
  constexpr int VPT = (VTASKS + NT - 1) / NT;
  static_assert(KT * CPR % NT == 0, "K tile must split evenly");

  __shared__ __align__(16) __bf16 Ks[KT * D];
  __shared__ __align__(16) __bf16 Vt[D * KT];

  int bid = blockIdx.x;
  const int tile = bid % a.tiles;
  bid /= a.tiles;
  const int qblk = bid % a.nq;
  const int bh = bid / a.nq;
  const int b = bh / a.Hh, h = bh - b * a.Hh;
  const BlockExt qe = block_ext(a, qblk);
  const int row0 = tile * RW;
  if (row0 >= qe.n) return;

  const int64_t in_off = (int64_t)b * a.sb + (int64_t)h * a.sh;
  const __bf16* qh = q + in_off;
  const __bf16* kh = k + in_off;
  const __bf16* vh = v + in_off;
  __bf16* oh = o + (int64_t)b * a.osb + (int64_t)h * a.osh;
  const int32_t* selrow = sel + ((int64_t)bh * a.nq + qblk) * a.topk;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, g = lane >> 5;
  const int wrow0 = row0 + wave * 32 * QB;
  const bool wave_active = wrow0 < qe.n;

  // ---- Q rows of this wave, in MFMA B-operand layout
  bf16x8 qreg[QB][D / 16];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int r = wrow0 + qb * 32 + l32;
    if (r < qe.n) {
      const __bf16* src = qh + (int64_t)slot_row(a, qe, r) * a.sn + 8 * g;
#pragma unroll
      for (int c = 0; c < D / 16; ++c) qreg[qb][c] = *reinterpret_cast<const bf16x8*>(src + 16 * c);
    } else {
#pragma unroll
      for (int c = 0; c < D / 16; ++c) qreg[qb][c] = bf16x8{};
    }
  }

  f32x16 oacc[QB][D / 32];
  float mrow[QB], lrow[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    mrow[qb] = -INFINITY;
    lrow[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[qb][db] = f32x16{};
  }

  // ---- kept-block walk state
  const int nkept = a.Pb + a.topk;
  auto kept_block = [&](int i) -> int {
    if (i < a.Pb) return i;
    int c = selrow[i - a.Pb];
    c = c < 0 ? 0 : (c >= a.nb ? a.nb - 1 : c);
    return a.Pb + c;
  };
  int bi = 0, kt = 0;
  BlockExt ke = block_ext(a, kept_block(0));

  u32x4 kbuf[KCH];
  u32x4 vbuf[VPT][4];

  auto load_tile = [&](const BlockExt& e, int t) {
    const int nv = min(KT, e.n - t * KT);
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int idx = tid + i * NT;
      const int key = idx / CPR, c = idx % CPR;
      if (key < nv) {
        const int row = slot_row(a, e, t * KT + key);
        kbuf[i] = *reinterpret_cast<const u32x4*>(kh + (int64_t)row * a.sn + c * 8);
      } else {
        kbuf[i] = u32x4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int task = tid + i * NT;
      const int grp = task / CPR, e8 = task % CPR;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = 4 * grp + j;
        if (task < VTASKS && key < nv) {
          const int row = slot_row(a, e, t * KT + key);
          vbuf[i][j] = *reinterpret_cast<const u32x4*>(vh + (int64_t)row * a.sn + e8 * 8);
        } else {
          vbuf[i][j] = u32x4{0, 0, 0, 0};
        }
      }
    }
  };

  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int idx = tid + i * NT;
      const int key = idx / CPR, c = idx % CPR;
      *reinterpret_cast<u32x4*>(Ks + key * D + ((c ^ (key & 7)) * 8)) = kbuf[i];
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int task = tid + i * NT;
      if (task < VTASKS) {
        const int grp = task / CPR, e8 = task % CPR;
        // position of the group's first key inside its permuted 16-key group
        const int p0 = 16 * (grp >> 2) + ((grp & 1) << 3) + ((grp & 2) << 1);
        const int pc = p0 >> 3, half = (p0 >> 2) & 1;
#pragma unroll
        for (int ii = 0; ii < 8; ++ii) {
          const int d = 8 * e8 + ii;
          const uint32_t s = (ii & 1) ? 0x07060302u : 0x05040100u;
          u32x2 w;
          w[0] = perm_b32(vbuf[i][1][ii >> 1], vbuf[i][0][ii >> 1], s);
          w[1] = perm_b32(vbuf[i][3][ii >> 1], vbuf[i][2][ii >> 1], s);
          *reinterpret_cast<u32x2*>(Vt + d * KT + ((pc ^ (d & 7)) * 8) + half * 4) = w;
        }
      }
    }
  };

  const float cexp = a.scale_log2e;
  load_tile(ke, kt);

#pragma unroll 1
  while (bi < nkept) {
    __syncthreads();
    store_tile();
    __syncthreads();
    const int nv = min(KT, ke.n - kt * KT);
    // advance and prefetch the next tile while this one is computed
    ++kt;
    if (kt * KT >= ke.n) {
      kt = 0;
      ++bi;
      if (bi < nkept) ke = block_ext(a, kept_block(bi));
    }
    if (bi < nkept) load_tile(ke, kt);

    if (wave_active) {
      f32x16 s[QB][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[qb][kb] = f32x16{};
        const int key = 32 * kb + l32;
#pragma unroll
        for (int c = 0; c < D / 16; ++c) {
          const int chunk = 2 * c + g;
          const bf16x8 kop = *reinterpret_cast<const bf16x8*>(Ks + key * D + ((chunk ^ (key & 7)) * 8));
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            s[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qreg[qb][c], s[qb][kb], 0, 0, 0);
        }
      }
      if (nv < KT) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3);
            if (key >= nv)
#pragma unroll
              for (int qb = 0; qb < QB; ++qb) s[qb][kb][r] = -INFINITY;
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
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int pc = 4 * kb + 2 * hh + g;
            const bf16x8 vop = *reinterpret_cast<const bf16x8*>(Vt + d * KT + ((pc ^ (d & 7)) * 8));
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
              oacc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pb[qb][kb][hh], oacc[qb][db], 0, 0, 0);
          }
      }
    }
  }

  // ---- normalise and store in raster order
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float ltot = lrow[qb] + __shfl_xor(lrow[qb], 32, 64);
    const float inv = 1.f / ltot;
    const int r = wrow0 + qb * 32 + l32;
    if (wave_active && r < qe.n) {
      __bf16* dst = oh + (int64_t)slot_row(a, qe, r) * a.osn + 4 * g;
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

template <int D, int NW, int QB>
hipError_t launch(const VsaArgs& a, const void* q, const void* k, const void* v, const int32_t* sel, void* o,
                  hipStream_t stream) {
  dim3 grid((int64_t)a.B * a.Hh * a.nq * a.tiles);
  hipLaunchKernelGGL((vsa_attend_kernel<D, NW, QB>), grid, dim3(NW * 64), 0, stream, a, (const __bf16*)q,
                     (const __bf16*)k, (const __bf16*)v, sel, (__bf16*)o);
  return hipGetLastError();
}

}  // namespace

hipError_t vsa_launch_attend(const VsaArgs& a, int variant, const void* q, const void* k, const void* v,
                             const int32_t* sel, void* o, hipStream_t stream) {
  if (a.D == 128) {
    if (variant == VSA_ATTEND_ROWS64) return launch<128, 2, 1>(a, q, k, v, sel, o, stream);
    return launch<128, 4, 1>(a, q, k, v, sel, o, stream);
  }
  if (variant == VSA_ATTEND_ROWS64) return launch<64, 2, 1>(a, q, k, v, sel, o, stream);
  return launch<64, 4, 1>(a, q, k, v, sel, o, stream);
}
