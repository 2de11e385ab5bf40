// Host-side geometry and validation for the block-sparse attention library.
// No HIP headers: this file builds and runs on any host.
//
// Geometry follows the "FastVideo VSA" user guide (vllm-omni docs): the
// latent grid is cut into spatiotemporal blocks (opening definition), the
// block count is the product of the per-axis block counts, e.g. 120 for the
// (31, 22, 40) grid in (4, 8, 8) blocks of the Wan routing log (section
// "Wan top-k behavior"), top-k must be positive and not above the block
// count (sections "Alternative configuration formats" and "Wan top-k
// behavior"), and prefix blocks have the cube's token count (section
// "Choose top-k": 64-token blocks that keep all prefix blocks).

#include <cstdint>
#include <cstdio>
#include <cmath>
#include <cstring>
#include <limits>

#include "vsa.h"
#include "vsa_limits.h"

namespace {

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool aligned16_elems(int64_t stride_elems) { return (stride_elems * 2) % 16 == 0; }

// Largest element offset touched for a [B][Hh][N][D] view with these strides.
bool span_fits(int64_t B, int64_t Hh, int64_t N, int64_t D, int64_t sb, int64_t sh,
               int64_t sn) {
  const int64_t lim = std::numeric_limits<int64_t>::max() / 4;
  if (sb > lim / (B > 0 ? B : 1) || sh > lim / (Hh > 0 ? Hh : 1) || sn > lim / (N > 0 ? N : 1))
    return false;
  return (B - 1) * sb + (Hh - 1) * sh + (N - 1) * sn + D < lim;
}

}  // namespace

extern "C" int vsa_plan(const vsa_problem* pr, vsa_plan_t* out) {
  if (pr == nullptr || out == nullptr) return VSA_ERR_INVALID_ARG;
  const vsa_problem& p = *pr;
  if (p.batch < 1 || p.heads < 1 || p.head_dim < 1 || p.prefix_len < 0) return VSA_ERR_INVALID_ARG;
  for (int a = 0; a < 3; ++a)
    if (p.latent[a] < 1 || p.cube[a] < 1) return VSA_ERR_INVALID_ARG;
  if (p.stride_b < 1 || p.stride_h < 1 || p.stride_n < 1 || p.o_stride_b < 1 ||
      p.o_stride_h < 1 || p.o_stride_n < 1)
    return VSA_ERR_INVALID_ARG;
  if (p.dtype != VSA_DTYPE_BF16 && p.dtype != VSA_DTYPE_F16) return VSA_ERR_UNSUPPORTED;
  if (p.head_dim != 64 && p.head_dim != 128) return VSA_ERR_UNSUPPORTED;

  const int64_t T = p.latent[0], H = p.latent[1], W = p.latent[2];
  const int64_t ct = p.cube[0], ch = p.cube[1], cw = p.cube[2];
  const int64_t nT = ceil_div(T, ct), nH = ceil_div(H, ch), nW = ceil_div(W, cw);
  const int64_t V = ct * ch * cw;
  if (V > VSA_MAX_CUBE_VOLUME) return VSA_ERR_UNSUPPORTED;
  const int64_t nb = nT * nH * nW;
  if (nb > VSA_MAX_BLOCKS) return VSA_ERR_UNSUPPORTED;
  if (ct > 1023 || ch > 1023 || cw > 1023) return VSA_ERR_UNSUPPORTED;
  const int64_t P = p.prefix_len;
  const int64_t Pb = ceil_div(P, V);
  const int64_t nq = Pb + nb;
  const int64_t N = P + T * H * W;
  if (N > (int64_t)INT32_MAX / 2) return VSA_ERR_OVERFLOW;
  if (p.topk < 1 || p.topk > nb) return VSA_ERR_TOPK;

  // q/k/v/o rows: the kernels keep a row's element offset inside one head in
  // 32 bits; the (b, h) base offset is 64-bit.
  const int64_t D = p.head_dim;
  if ((N - 1) * p.stride_n + D > (int64_t)INT32_MAX) return VSA_ERR_OVERFLOW;
  if ((N - 1) * p.o_stride_n + D > (int64_t)INT32_MAX) return VSA_ERR_OVERFLOW;
  if (!span_fits(p.batch, p.heads, N, D, p.stride_b, p.stride_h, p.stride_n) ||
      !span_fits(p.batch, p.heads, N, D, p.o_stride_b, p.o_stride_h, p.o_stride_n))
    return VSA_ERR_OVERFLOW;
  if (!aligned16_elems(p.stride_b) || !aligned16_elems(p.stride_h) || !aligned16_elems(p.stride_n) ||
      !aligned16_elems(p.o_stride_b) || !aligned16_elems(p.o_stride_h) ||
      !aligned16_elems(p.o_stride_n))
    return VSA_ERR_ALIGN;
  // output rows must not overlap (each token row is written by one lane pair)
  if (p.o_stride_n < D) return VSA_ERR_INVALID_ARG;

  const int64_t BH = (int64_t)p.batch * p.heads;
  const int64_t sel_elems = BH * nq * p.topk;
  if (sel_elems > (int64_t)INT32_MAX) return VSA_ERR_OVERFLOW;

  vsa_plan_t r;
  std::memset(&r, 0, sizeof(r));
  r.p = p;
  r.nblk[0] = (int32_t)nT;
  r.nblk[1] = (int32_t)nH;
  r.nblk[2] = (int32_t)nW;
  r.num_blocks = (int32_t)nb;
  r.num_prefix_blocks = (int32_t)Pb;
  r.num_q_blocks = (int32_t)nq;
  r.cube_volume = (int32_t)V;
  r.seq_len = N;
  const int64_t qbar_bytes = BH * nq * D * 4;
  r.kbar_offset = ceil_div(qbar_bytes, 256) * 256;
  r.workspace_bytes = r.kbar_offset + BH * nb * D * 4;
  r.sel_elems = sel_elems;
  r.scale = (float)(1.0 / std::sqrt((double)D));

  // Score/top-k tiling: rows of the per-row score buffer live in LDS
  // (4 bytes per cube and row); keep it within the budget and prefer enough
  // workgroups to cover the machine.
  // Up to VSA_SELECT_MFMA_MAX_BLOCKS cubes the matrix-core kernel takes 16
  // rows per workgroup.
  int rows = VSA_SELECT_MAX_ROWS;
  if (nb > VSA_SELECT_MFMA_MAX_BLOCKS) {
    while (rows > 1 && (int64_t)rows * nb * 4 > VSA_SELECT_SCORE_LDS) rows /= 2;
    while (rows > 4 && BH * ceil_div(nq, rows) < 1024) rows /= 2;
  }
  r.select_rows = rows;

  // Attention tiling: query rows per workgroup by cube volume.
  if (V <= 64) {
    r.attend_variant = VSA_ATTEND_ROWS64;
    r.attend_tiles = 1;
  } else {
    r.attend_variant = VSA_ATTEND_ROWS256;
    r.attend_tiles = (int32_t)ceil_div(V, 256);
  }
  const int64_t grid = BH * nq * r.attend_tiles;
  if (grid > (int64_t)INT32_MAX) return VSA_ERR_OVERFLOW;
  *out = r;
  return VSA_OK;
}

extern "C" int vsa_describe(const vsa_plan_t* plan, char* buf, size_t len) {
  if (plan == nullptr || (buf == nullptr && len > 0)) return VSA_ERR_INVALID_ARG;
  const vsa_problem& p = plan->p;
  const double keep = plan->num_blocks > 0 ? 100.0 * p.topk / plan->num_blocks : 0.0;
  char tmp[512];
  int n = std::snprintf(tmp, sizeof(tmp),
                        "seq_len=%lld, dit_seq_shape=(%d, %d, %d), block_size=(%d, %d, %d), "
                        "num_blocks=%d, topk=%d, keep_ratio=%.1f%%",
                        (long long)plan->seq_len, p.latent[0], p.latent[1], p.latent[2], p.cube[0],
                        p.cube[1], p.cube[2], plan->num_blocks, p.topk, keep);
  if (n < 0) return VSA_ERR_INVALID_ARG;
  if (len > 0) {
    size_t c = (size_t)n < len - 1 ? (size_t)n : len - 1;
    std::memcpy(buf, tmp, c);
    buf[c] = '\0';
  }
  return n;
}

extern "C" const char* vsa_status_str(int s) {
  switch (s) {
    case VSA_OK: return "ok";
    case VSA_ERR_INVALID_ARG: return "invalid argument";
    case VSA_ERR_TOPK: return "topk must be in 1..num_blocks";
    case VSA_ERR_UNSUPPORTED: return "unsupported head_dim, dtype or size";
    case VSA_ERR_ALIGN: return "pointer or stride not 16-byte aligned";
    case VSA_ERR_OVERFLOW: return "offsets or counts overflow the kernels' index range";
    case VSA_ERR_DEVICE: return "current device is not gfx950 or a device query failed";
    case VSA_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}
