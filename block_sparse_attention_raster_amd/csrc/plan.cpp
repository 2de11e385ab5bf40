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
// "Choose top-k": 64-token blocks that keep all prefix blocks). q and k/v may
// lie on different grids with different cube shapes, and a sparsity maps to
// a top-k (the "fastbsa" package page, section "Use").

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cmath>
#include <cstring>
#include <limits>

#include "vsa.h"
#include "vsa_limits.h"

namespace {

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Largest (N_k - 1) * kv_stride_n + head_dim: 2^32 - 64 bytes.
constexpr int64_t kKvSpanElems = 0x7FFFFFE0;

bool aligned16_elems(int64_t stride_elems) { return (stride_elems * 2) % 16 == 0; }

// Largest element offset touched for a [B][Hh][N][D] view with these strides.
bool span_fits(int64_t B, int64_t Hh, int64_t N, int64_t D, int64_t sb, int64_t sh,
               int64_t sn) {
  const int64_t lim = std::numeric_limits<int64_t>::max() / 4;
  if (sb > lim / (B > 0 ? B : 1) || sh > lim / (Hh > 0 ? Hh : 1) || sn > lim / (N > 0 ? N : 1))
    return false;
  return (B - 1) * sb + (Hh - 1) * sh + (N - 1) * sn + D < lim;
}

// One side's grid cut into blocks (q's or k/v's).
struct Side {
  int64_t T, H, W, ct, ch, cw;
  int64_t nT, nH, nW, V, nb, Pb, N;
};

int derive_side(const int32_t* latent, const int32_t* cube, int64_t P, Side& s) {
  s.T = latent[0];
  s.H = latent[1];
  s.W = latent[2];
  s.ct = cube[0];
  s.ch = cube[1];
  s.cw = cube[2];
  if (s.T < 1 || s.H < 1 || s.W < 1 || s.ct < 1 || s.ch < 1 || s.cw < 1) return VSA_ERR_INVALID_ARG;
  s.nT = ceil_div(s.T, s.ct);
  s.nH = ceil_div(s.H, s.ch);
  s.nW = ceil_div(s.W, s.cw);
  s.V = s.ct * s.ch * s.cw;
  if (s.ct > 1023 || s.ch > 1023 || s.cw > 1023) return VSA_ERR_UNSUPPORTED;
  if (s.V > VSA_MAX_CUBE_VOLUME) return VSA_ERR_UNSUPPORTED;
  s.nb = s.nT * s.nH * s.nW;
  if (s.nb > VSA_MAX_BLOCKS) return VSA_ERR_UNSUPPORTED;
  s.Pb = ceil_div(P, s.V);
  s.N = P + s.T * s.H * s.W;
  if (s.N > (int64_t)INT32_MAX / 2) return VSA_ERR_OVERFLOW;
  return VSA_OK;
}

// A group of n values is either all zero (unset) or all >= 1.
template <typename T>
int group_state(const T* v, int n) {  // 0 unset, 1 set, -1 invalid
  int zeros = 0, pos = 0;
  for (int i = 0; i < n; ++i) {
    zeros += v[i] == 0;
    pos += v[i] >= 1;
  }
  return zeros == n ? 0 : pos == n ? 1 : -1;
}

// Row offsets of a [B][Hh][N][D] view: within a head in 32 bits, overall in
// 64 bits, and 16-byte aligned.
int check_view(int64_t B, int64_t Hh, int64_t N, int64_t D, int64_t sb, int64_t sh, int64_t sn) {
  if ((N - 1) * sn + D > (int64_t)INT32_MAX) return VSA_ERR_OVERFLOW;
  if (!span_fits(B, Hh, N, D, sb, sh, sn)) return VSA_ERR_OVERFLOW;
  if (!aligned16_elems(sb) || !aligned16_elems(sh) || !aligned16_elems(sn)) return VSA_ERR_ALIGN;
  return VSA_OK;
}

}  // namespace

extern "C" int vsa_plan(const vsa_problem* pr, vsa_plan_t* out) {
  if (pr == nullptr || out == nullptr) return VSA_ERR_INVALID_ARG;
  vsa_problem p = *pr;
  if (p.batch < 1 || p.heads < 1 || p.head_dim < 1 || p.prefix_len < 0) return VSA_ERR_INVALID_ARG;
  for (int a = 0; a < 3; ++a)
    if (p.latent[a] < 1 || p.cube[a] < 1) return VSA_ERR_INVALID_ARG;
  // Stride groups are all zero (a default) or all >= 1. Defaults: q
  // contiguous [B][Hh][N][D]; o as q; k and v as q on q's grid, else
  // contiguous on their own grid.
  const int64_t qs[3] = {p.stride_b, p.stride_h, p.stride_n};
  const int64_t os[3] = {p.o_stride_b, p.o_stride_h, p.o_stride_n};
  const int64_t kvs[3] = {p.kv_stride_b, p.kv_stride_h, p.kv_stride_n};
  const int gq = group_state(qs, 3), go = group_state(os, 3);
  const int gl = group_state(p.latent_k, 3), gc = group_state(p.cube_k, 3), gs = group_state(kvs, 3);
  if (gq < 0 || go < 0 || gl < 0 || gc < 0 || gs < 0) return VSA_ERR_INVALID_ARG;
  if (gl == 0) std::memcpy(p.latent_k, p.latent, sizeof(p.latent));
  if (gc == 0) std::memcpy(p.cube_k, p.cube, sizeof(p.cube));
  const int64_t nq_tok = (int64_t)p.prefix_len + (int64_t)p.latent[0] * p.latent[1] * p.latent[2];
  const int64_t nk_tok = (int64_t)p.prefix_len + (int64_t)p.latent_k[0] * p.latent_k[1] * p.latent_k[2];
  if (gq == 0) {
    p.stride_n = p.head_dim;
    p.stride_h = nq_tok * p.head_dim;
    p.stride_b = (int64_t)p.heads * nq_tok * p.head_dim;
  }
  if (go == 0) {
    p.o_stride_b = p.stride_b;
    p.o_stride_h = p.stride_h;
    p.o_stride_n = p.stride_n;
  }
  if (gs == 0) {
    const bool same_grid = std::memcmp(p.latent_k, p.latent, sizeof(p.latent)) == 0;
    p.kv_stride_n = same_grid ? p.stride_n : p.head_dim;
    p.kv_stride_h = same_grid ? p.stride_h : nk_tok * p.head_dim;
    p.kv_stride_b = same_grid ? p.stride_b : (int64_t)p.heads * nk_tok * p.head_dim;
  }
  if (p.dtype != VSA_DTYPE_BF16 && p.dtype != VSA_DTYPE_F16) return VSA_ERR_UNSUPPORTED;
  if (p.head_dim != 64 && p.head_dim != 128) return VSA_ERR_UNSUPPORTED;

  const int64_t P = p.prefix_len;
  Side q, k;
  int st = derive_side(p.latent, p.cube, P, q);
  if (st != VSA_OK) return st;
  if ((st = derive_side(p.latent_k, p.cube_k, P, k)) != VSA_OK) return st;
  const int64_t nq = q.Pb + q.nb;
  const int64_t nb = k.nb;
  if (p.topk < 1 || p.topk > nb) return VSA_ERR_TOPK;

  // q/k/v/o rows: the kernels keep a row's element offset inside one head in
  // 32 bits; the (b, h) base offset is 64-bit.
  const int64_t D = p.head_dim;
  const int64_t B = p.batch, Hh = p.heads;
  if ((st = check_view(B, Hh, q.N, D, p.stride_b, p.stride_h, p.stride_n)) != VSA_OK) return st;
  if ((st = check_view(B, Hh, q.N, D, p.o_stride_b, p.o_stride_h, p.o_stride_n)) != VSA_OK) return st;
  if ((st = check_view(B, Hh, k.N, D, p.kv_stride_b, p.kv_stride_h, p.kv_stride_n)) != VSA_OK) return st;
  // k/v rows are addressed by byte offsets from the head's first row, and
  // offsets from 2^32 - 64 up mark tail slots: a head's k/v byte span stays
  // below that
  if ((k.N - 1) * p.kv_stride_n + D > kKvSpanElems) return VSA_ERR_OVERFLOW;
  // output rows must not overlap (each token row is written by one lane pair)
  if (p.o_stride_n < D) return VSA_ERR_INVALID_ARG;

  const int64_t BH = B * Hh;
  const int64_t sel_elems = BH * nq * p.topk;
  if (sel_elems > (int64_t)INT32_MAX) return VSA_ERR_OVERFLOW;

  vsa_plan_t r;
  std::memset(&r, 0, sizeof(r));
  r.p = p;
  r.nblk[0] = (int32_t)q.nT;
  r.nblk[1] = (int32_t)q.nH;
  r.nblk[2] = (int32_t)q.nW;
  r.num_blocks = (int32_t)nb;
  r.num_prefix_blocks = (int32_t)q.Pb;
  r.num_q_blocks = (int32_t)nq;
  r.cube_volume = (int32_t)q.V;
  r.seq_len = q.N;
  r.nblk_k[0] = (int32_t)k.nT;
  r.nblk_k[1] = (int32_t)k.nH;
  r.nblk_k[2] = (int32_t)k.nW;
  r.num_prefix_blocks_k = (int32_t)k.Pb;
  r.cube_volume_k = (int32_t)k.V;
  r.seq_len_k = k.N;
  const int64_t qbar_bytes = BH * nq * D * 4;
  r.kbar_offset = ceil_div(qbar_bytes, 256) * 256;
  r.workspace_bytes = r.kbar_offset + BH * nb * D * 4;
  r.sel_elems = sel_elems;
  r.scale = (float)(1.0 / std::sqrt((double)D));

  // Score/top-k tiling: rows of the per-row score buffer live in LDS
  // (4 bytes per cube and row); keep it within the budget and prefer enough
  // workgroups to cover the machine.
  // Up to VSA_SELECT_MFMA_MAX_BLOCKS cubes the matrix-core kernel takes 16
  // or 32 rows per workgroup (its launcher decides by LDS and grid size).
  int rows = VSA_SELECT_MAX_ROWS;
  if (nb > VSA_SELECT_MFMA_MAX_BLOCKS) {
    while (rows > 1 && (int64_t)rows * nb * 4 > VSA_SELECT_SCORE_LDS) rows /= 2;
    while (rows > 4 && BH * ceil_div(nq, rows) < 1024) rows /= 2;
  }
  r.select_rows = rows;

  // Attention tiling: query rows per workgroup by the query cube volume.
  if (q.V <= 64) {
    r.attend_variant = VSA_ATTEND_ROWS64;
    r.attend_tiles = 1;
  } else {
    r.attend_variant = VSA_ATTEND_ROWS256;
    r.attend_tiles = (int32_t)ceil_div(q.V, 256);
  }
  const int64_t grid = BH * nq * r.attend_tiles;
  if (grid > (int64_t)INT32_MAX) return VSA_ERR_OVERFLOW;
  *out = r;
  return VSA_OK;
}

extern "C" int vsa_topk_for_sparsity(int32_t num_blocks, double sparsity) {
  if (num_blocks < 1 || !(sparsity >= 0.0 && sparsity < 1.0)) return VSA_ERR_INVALID_ARG;
  // floor(nb * (1 - s)); a product within 1e-9 (relative) of an integer is
  // that integer, since decimal sparsities are not exact in binary (e.g.
  // 120 * (1 - 0.9) evaluates to 11.999999999999998)
  const double x = (double)num_blocks * (1.0 - sparsity);
  const double n = std::nearbyint(x);
  const double keep = std::fabs(x - n) <= 1e-9 * std::fmax(1.0, x) ? n : std::floor(x);
  if (keep < 1.0) return 1;
  if (keep > (double)num_blocks) return num_blocks;
  return (int)keep;
}

extern "C" int vsa_block_counts(const vsa_plan_t* plan, int32_t side, int32_t* counts, int64_t len) {
  if (plan == nullptr || (side != VSA_SIDE_Q && side != VSA_SIDE_K) || len < 0 || (counts == nullptr && len > 0))
    return VSA_ERR_INVALID_ARG;
  const vsa_problem& p = plan->p;
  const int32_t* latent = side == VSA_SIDE_Q ? p.latent : p.latent_k;
  const int32_t* cube = side == VSA_SIDE_Q ? p.cube : p.cube_k;
  Side g;
  const int st = derive_side(latent, cube, p.prefix_len, g);
  if (st != VSA_OK) return st;
  const int64_t total = g.Pb + g.nb;
  if (counts != nullptr) {
    int64_t i = 0;
    // prefix blocks: V tokens each, the last one the remainder
    for (int64_t b = 0; b < g.Pb && i < len; ++b, ++i) {
      const int64_t rest = (int64_t)p.prefix_len - b * g.V;
      counts[i] = (int32_t)(rest < g.V ? rest : g.V);
    }
    // cubes in raster order of the cube grid: the product over the axes of
    // the cube's extent clipped to the grid
    for (int64_t c = 0; c < g.nb && i < len; ++c, ++i) {
      const int64_t bw = c % g.nW, bh = (c / g.nW) % g.nH, bt = c / (g.nW * g.nH);
      const int64_t et = std::min(g.ct, g.T - bt * g.ct), eh = std::min(g.ch, g.H - bh * g.ch),
                    ew = std::min(g.cw, g.W - bw * g.cw);
      counts[i] = (int32_t)(et * eh * ew);
    }
  }
  return (int)total;
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
  const bool own_k = std::memcmp(p.latent_k, p.latent, sizeof(p.latent)) != 0 ||
                     std::memcmp(p.cube_k, p.cube, sizeof(p.cube)) != 0;
  if (own_k) {  // key side of a two-grid problem
    const int m = std::snprintf(tmp + n, sizeof(tmp) - (size_t)n,
                                ", kv_seq_len=%lld, kv_seq_shape=(%d, %d, %d), kv_block_size=(%d, %d, %d)",
                                (long long)plan->seq_len_k, p.latent_k[0], p.latent_k[1], p.latent_k[2],
                                p.cube_k[0], p.cube_k[1], p.cube_k[2]);
    if (m < 0) return VSA_ERR_INVALID_ARG;
    n += m;
  }
  if (len > 0) {
    size_t c = (size_t)n < len - 1 ? (size_t)n : len - 1;
    std::memcpy(buf, tmp, c);
    buf[c] = '\0';
  }
  return n;
}

extern "C" int vsa_route(const vsa_problem* pr, int32_t checkpoint_mode, vsa_route_t* out) {
  if (pr == nullptr || out == nullptr) return VSA_ERR_INVALID_ARG;
  if (checkpoint_mode != VSA_CHECKPOINT_NATIVE && checkpoint_mode != VSA_CHECKPOINT_DMD)
    return VSA_ERR_INVALID_ARG;
  if (pr->topk < 1) return VSA_ERR_TOPK;
  vsa_route_t r;
  std::memset(&r, 0, sizeof(r));
  r.checkpoint_mode = checkpoint_mode;
  r.topk = pr->topk;
  vsa_problem p = *pr;
  int st = vsa_plan(&p, &r.plan);
  if (st == VSA_ERR_TOPK) {
    // topk above the block count: plan with every block for the geometry
    p.topk = 1;
    if (vsa_plan(&p, &r.plan) == VSA_OK) {
      p.topk = r.plan.num_blocks;
      st = vsa_plan(&p, &r.plan);
      r.has_plan = st == VSA_OK;
      r.route = VSA_ROUTE_DENSE;
      r.reason = VSA_REASON_TOPK_ABOVE_BLOCKS;
      *out = r;
      return VSA_OK;
    }
    st = vsa_plan(&p, &r.plan);   // the shape itself is refused
  }
  if (st != VSA_OK) {
    std::memset(&r.plan, 0, sizeof(r.plan));
    r.route = VSA_ROUTE_DENSE;
    r.reason = VSA_REASON_UNSUPPORTED;
    r.status = st;
    *out = r;
    return VSA_OK;
  }
  r.has_plan = 1;
  if (pr->topk == r.plan.num_blocks) {
    if (checkpoint_mode == VSA_CHECKPOINT_NATIVE) {
      r.route = VSA_ROUTE_DENSE;
      r.reason = VSA_REASON_ALL_BLOCKS_NATIVE;
    } else {
      r.route = VSA_ROUTE_VSA_ALL_BLOCKS;
    }
  } else {
    r.route = VSA_ROUTE_VSA;
  }
  *out = r;
  return VSA_OK;
}

extern "C" int vsa_describe_route(const vsa_route_t* r, char* buf, size_t len) {
  if (r == nullptr || (buf == nullptr && len > 0)) return VSA_ERR_INVALID_ARG;
  static const char* const kRoute[] = {"VSA", "VSA_ALL_BLOCKS", "SDPA"};
  static const char* const kMode[] = {"native", "dmd"};
  static const char* const kReason[] = {"", "topk > num_blocks for the runtime shape",
                                        "topk == num_blocks on a native checkpoint",
                                        "unsupported problem: "};
  if (r->route < 0 || r->route > 2 || r->checkpoint_mode < 0 || r->checkpoint_mode > 1 || r->reason < 0 ||
      r->reason > 3)
    return VSA_ERR_INVALID_ARG;
  char tmp[768];
  int n = 0;
  if (r->has_plan) {
    const vsa_plan_t& pl = r->plan;
    const vsa_problem& p = pl.p;
    const double keep = 100.0 * r->topk / pl.num_blocks;
    n = std::snprintf(tmp, sizeof(tmp),
                      "FASTVIDEO_VSA routing: seq_len=%lld, dit_seq_shape=(%d, %d, %d), block_size=(%d, %d, %d), "
                      "num_blocks=%d, topk=%d, keep_ratio=%.1f%%, checkpoint_mode=%s, route=%s",
                      (long long)pl.seq_len, p.latent[0], p.latent[1], p.latent[2], p.cube[0], p.cube[1],
                      p.cube[2], pl.num_blocks, r->topk, keep, kMode[r->checkpoint_mode], kRoute[r->route]);
  } else {
    n = std::snprintf(tmp, sizeof(tmp), "FASTVIDEO_VSA routing: topk=%d, checkpoint_mode=%s, route=%s", r->topk,
                      kMode[r->checkpoint_mode], kRoute[r->route]);
  }
  if (n < 0) return VSA_ERR_INVALID_ARG;
  if (r->reason != VSA_REASON_NONE) {
    const int m = std::snprintf(tmp + n, sizeof(tmp) - (size_t)n, ", reason=%s%s", kReason[r->reason],
                                r->reason == VSA_REASON_UNSUPPORTED ? vsa_status_str(r->status) : "");
    if (m < 0) return VSA_ERR_INVALID_ARG;
    n += m;
  }
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
    case VSA_ERR_SCRATCH: return "problem needs more scratch than the allocation-free entry point holds (32 MiB)";
    default: return "unknown status";
  }
}
