// extern "C" entry points of the block-sparse attention library: argument
// checks, the gfx950 device check and kernel launches on the caller's
// stream. No allocation, no synchronisation.

#include <atomic>
#include <cstring>

#include "vsa.h"
#include "vsa_device.h"
#include "vsa_limits.h"

hipError_t vsa_launch_pool(const VsaArgs& a, const void* q, const void* k, float* qbar, float* kbar,
                           hipStream_t stream);
hipError_t vsa_launch_score_topk(const VsaArgs& a, const float* qbar, const float* kbar, int32_t* sel,
                                 hipStream_t stream);
hipError_t vsa_launch_attend(const VsaArgs& a, int variant, const void* q, const void* k, const void* v,
                             const int32_t* sel, void* o, hipStream_t stream);

// Scratch memory of vsa_forward_noalloc: the pooled means (qbar, kbar) in a
// fixed device array, so that the call allocates nothing. Each device holds
// its own copy from the library's load until the process ends. In host code
// `scratch` names a host-side stand-in, never device memory: the device
// address comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) unsigned char scratch[VSA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];  // 0 unknown, 1 gfx950, -1 other

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return VSA_ERR_DEVICE;
  if (dev < kMaxDevices) {
    const int known = g_arch_ok[dev].load(std::memory_order_relaxed);
    if (known != 0) return known > 0 ? VSA_OK : VSA_ERR_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return VSA_ERR_DEVICE;
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < kMaxDevices) g_arch_ok[dev].store(ok ? 1 : -1, std::memory_order_relaxed);
  return ok ? VSA_OK : VSA_ERR_DEVICE;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Re-validates a caller-held plan (it is plain data and could be edited) by
// planning its problem again and comparing the derived fields.
int check_plan(const vsa_plan_t* plan) {
  if (plan == nullptr) return VSA_ERR_INVALID_ARG;
  vsa_plan_t fresh;
  const int st = vsa_plan(&plan->p, &fresh);
  if (st != VSA_OK) return st;
  const bool same =
      fresh.nblk[0] == plan->nblk[0] && fresh.nblk[1] == plan->nblk[1] && fresh.nblk[2] == plan->nblk[2] &&
      fresh.num_blocks == plan->num_blocks && fresh.num_prefix_blocks == plan->num_prefix_blocks &&
      fresh.num_q_blocks == plan->num_q_blocks && fresh.cube_volume == plan->cube_volume &&
      fresh.seq_len == plan->seq_len && fresh.workspace_bytes == plan->workspace_bytes &&
      fresh.kbar_offset == plan->kbar_offset && fresh.sel_elems == plan->sel_elems &&
      fresh.scale == plan->scale && fresh.select_rows == plan->select_rows &&
      fresh.attend_variant == plan->attend_variant && fresh.attend_tiles == plan->attend_tiles &&
      fresh.nblk_k[0] == plan->nblk_k[0] && fresh.nblk_k[1] == plan->nblk_k[1] &&
      fresh.nblk_k[2] == plan->nblk_k[2] && fresh.num_prefix_blocks_k == plan->num_prefix_blocks_k &&
      fresh.cube_volume_k == plan->cube_volume_k && fresh.seq_len_k == plan->seq_len_k &&
      std::memcmp(&fresh.p, &plan->p, sizeof(vsa_problem)) == 0;
  return same ? VSA_OK : VSA_ERR_INVALID_ARG;
}

uint64_t magic(int64_t d) { return ((1ull << 32) + (uint64_t)d - 1) / (uint64_t)d; }

VsaGrid make_grid(const int32_t* latent, const int32_t* cube, const int32_t* nblk, int32_t P, int32_t V,
                  int32_t Pb) {
  VsaGrid g;
  std::memset(&g, 0, sizeof(g));
  g.T = latent[0];
  g.H = latent[1];
  g.W = latent[2];
  g.ct = cube[0];
  g.ch = cube[1];
  g.cw = cube[2];
  g.nT = nblk[0];
  g.nH = nblk[1];
  g.nW = nblk[2];
  g.P = P;
  g.V = V;
  g.Pb = Pb;
  g.nb = g.nT * g.nH * g.nW;
  g.magic_nW = magic(g.nW);
  g.magic_nH = magic(g.nH);
  const int64_t tail_h = g.H - (int64_t)(g.nH - 1) * g.ch, tail_w = g.W - (int64_t)(g.nW - 1) * g.cw;
  const int64_t ehs[2] = {g.ch, tail_h}, ews[2] = {g.cw, tail_w};
  for (int iw = 0; iw < 2; ++iw) g.magic_ew[iw] = magic(ews[iw]);
  for (int ih = 0; ih < 2; ++ih)
    for (int iw = 0; iw < 2; ++iw) g.magic_ehw[2 * ih + iw] = magic(ehs[ih] * ews[iw]);
  return g;
}

VsaArgs make_args(const vsa_plan_t& pl) {
  const vsa_problem& p = pl.p;
  VsaArgs a;
  std::memset(&a, 0, sizeof(a));
  a.B = p.batch;
  a.Hh = p.heads;
  a.D = p.head_dim;
  a.gq = make_grid(p.latent, p.cube, pl.nblk, p.prefix_len, pl.cube_volume, pl.num_prefix_blocks);
  a.gk = make_grid(p.latent_k, p.cube_k, pl.nblk_k, p.prefix_len, pl.cube_volume_k, pl.num_prefix_blocks_k);
  a.nq = pl.num_q_blocks;
  a.nb = pl.num_blocks;
  a.topk = p.topk;
  a.sb = p.stride_b;
  a.sh = p.stride_h;
  a.sn = (int32_t)p.stride_n;
  a.ksb = p.kv_stride_b;
  a.ksh = p.kv_stride_h;
  a.ksn = (int32_t)p.kv_stride_n;
  a.osb = p.o_stride_b;
  a.osh = p.o_stride_h;
  a.osn = (int32_t)p.o_stride_n;
  a.scale_log2e = pl.scale * 1.4426950408889634f;
  a.select_rows = pl.select_rows;
  a.tiles = pl.attend_tiles;
  a.f16 = p.dtype == VSA_DTYPE_F16;
  return a;
}

}  // namespace

extern "C" int vsa_pool(const vsa_plan_t* plan, const void* q, const void* k, void* workspace, void* stream) {
  int st = check_plan(plan);
  if (st != VSA_OK) return st;
  if (q == nullptr || k == nullptr || workspace == nullptr) return VSA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return VSA_ERR_ALIGN;
  if ((st = check_device()) != VSA_OK) return st;
  const VsaArgs a = make_args(*plan);
  float* qbar = static_cast<float*>(workspace);
  float* kbar = reinterpret_cast<float*>(static_cast<char*>(workspace) + plan->kbar_offset);
  if (vsa_launch_pool(a, q, k, qbar, kbar, static_cast<hipStream_t>(stream)) != hipSuccess) return VSA_ERR_LAUNCH;
  return VSA_OK;
}

extern "C" int vsa_score_topk(const vsa_plan_t* plan, const void* workspace, int32_t* sel, void* stream) {
  int st = check_plan(plan);
  if (st != VSA_OK) return st;
  if (workspace == nullptr || sel == nullptr) return VSA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0 || (reinterpret_cast<uintptr_t>(sel) & 3u) != 0)
    return VSA_ERR_ALIGN;
  if ((st = check_device()) != VSA_OK) return st;
  const VsaArgs a = make_args(*plan);
  const float* qbar = static_cast<const float*>(workspace);
  const float* kbar = reinterpret_cast<const float*>(static_cast<const char*>(workspace) + plan->kbar_offset);
  if (vsa_launch_score_topk(a, qbar, kbar, sel, static_cast<hipStream_t>(stream)) != hipSuccess)
    return VSA_ERR_LAUNCH;
  return VSA_OK;
}

extern "C" int vsa_select(const vsa_plan_t* plan, const void* q, const void* k, void* workspace,
                          int32_t* sel, void* stream) {
  if (q == nullptr || k == nullptr || workspace == nullptr || sel == nullptr) return VSA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(sel) & 3u) != 0) return VSA_ERR_ALIGN;
  const int st = vsa_pool(plan, q, k, workspace, stream);
  if (st != VSA_OK) return st;
  return vsa_score_topk(plan, workspace, sel, stream);
}

extern "C" int vsa_attend(const vsa_plan_t* plan, const void* q, const void* k, const void* v,
                          const int32_t* sel, void* o, void* stream) {
  int st = check_plan(plan);
  if (st != VSA_OK) return st;
  if (q == nullptr || k == nullptr || v == nullptr || sel == nullptr || o == nullptr)
    return VSA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      (reinterpret_cast<uintptr_t>(sel) & 3u) != 0)
    return VSA_ERR_ALIGN;
  if ((st = check_device()) != VSA_OK) return st;
  const VsaArgs a = make_args(*plan);
  if (vsa_launch_attend(a, plan->attend_variant, q, k, v, sel, o, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return VSA_ERR_LAUNCH;
  return VSA_OK;
}

extern "C" int vsa_forward(const vsa_plan_t* plan, const void* q, const void* k, const void* v,
                           void* workspace, int32_t* sel, void* o, void* stream) {
  const int st = vsa_select(plan, q, k, workspace, sel, stream);
  if (st != VSA_OK) return st;
  return vsa_attend(plan, q, k, v, sel, o, stream);
}

namespace {

// Device address of `scratch` on each device, looked up once per device
// with that device current (0: not yet).
std::atomic<uintptr_t> g_scratch[kMaxDevices];

int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return VSA_ERR_DEVICE;
  uintptr_t p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == 0) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();   // leave no error behind for the caller's next HIP call
      return VSA_ERR_DEVICE;
    }
    p = reinterpret_cast<uintptr_t>(ptr);
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = reinterpret_cast<void*>(p);
  return VSA_OK;
}

}  // namespace

extern "C" int vsa_forward_noalloc(const vsa_plan_t* plan, const void* q, const void* k, const void* v,
                                   int32_t* sel, void* o, void* stream) {
  int st = check_plan(plan);
  if (st != VSA_OK) return st;
  if (plan->workspace_bytes > (int64_t)VSA_NOALLOC_SCRATCH_BYTES) return VSA_ERR_SCRATCH;
  if (q == nullptr || k == nullptr || v == nullptr || sel == nullptr || o == nullptr) return VSA_ERR_INVALID_ARG;
  if ((st = check_device()) != VSA_OK) return st;
  void* ws = nullptr;
  if ((st = scratch_address(&ws)) != VSA_OK) return st;
  // every element of qbar and kbar is written by the pooling kernel before
  // it is read, so the array's previous contents need no clearing
  return vsa_forward(plan, q, k, v, ws, sel, o, stream);
}
