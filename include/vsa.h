/*
 * vsa.h - C ABI of a top-k block-sparse attention library for AMD Instinct
 * MI355X (gfx950) over a raster-ordered (T, H, W) video latent grid.
 *
 * The operation (pages: "FastVideo VSA" user guide of vllm-omni, opening
 * definition and section "Wan top-k behavior"; "fastbsa" package page,
 * sections "Use" and "How it works"):
 *
 *   The N = P + T*H*W tokens of each (batch, head) are q, k, v rows in
 *   raster order: P optional prefix tokens first, then grid point (t, h, w)
 *   at row P + (t*H + h)*W + w. The grid is cut into cubes of ct x ch x cw
 *   tokens (cubes at the far edge of an axis hold fewer), numbered in raster
 *   order of the cube grid; the prefix forms ceil(P / V) blocks of
 *   V = ct*ch*cw tokens, always kept. Every query block (prefix blocks first,
 *   then cubes) is scored against every cube by
 *       s[i][j] = mean_q(i) . mean_k(j) * head_dim^-1/2
 *   (means over the block's valid tokens), keeps its topk highest-scoring
 *   cubes (equal scores: lower cube id first), and each of its query tokens
 *   runs exact softmax attention, scale head_dim^-1/2, over the tokens of
 *   the kept cubes and of all prefix blocks.
 *
 * Data types and layouts
 *   q, k, v, o   bfloat16 or float16 (plan dtype; the user guide, section
 *                "Verify routing and fallback": the Wan route takes FP16
 *                or BF16), element (b, h, n, d) at
 *                b*stride_b + h*stride_h + n*stride_n + d   (elements);
 *                d is contiguous. q, k and v share one set of strides
 *                unless kv_stride_* are given; o has its own. Base pointers
 *                and strides*2 must be multiples of 16 bytes. With a key
 *                grid of its own, k and v hold N_k = P + T_k*H_k*W_k rows
 *                in raster order of that grid. Within one (b, h):
 *                (N-1)*stride_n + head_dim <= 2^31 - 1 for q and o, and
 *                (N_k-1)*kv_stride_n + head_dim <= 2^31 - 32 for k and v,
 *                else VSA_ERR_OVERFLOW.
 *   workspace    float32 pooled means, written by vsa_select:
 *                  qbar [B][Hh][num_q_blocks][head_dim], then
 *                  kbar [B][Hh][num_blocks][head_dim] at byte offset
 *                  plan.kbar_offset. Size plan.workspace_bytes.
 *   sel          int32 [B][Hh][num_q_blocks][topk], ascending cube ids in
 *                0 .. num_blocks-1. Prefix blocks are kept implicitly and
 *                never appear in sel.
 *
 * Ownership and execution
 *   The caller allocates and owns every buffer (device memory for q, k, v,
 *   o, sel and workspace; host memory for the problem and plan structs).
 *   The library allocates nothing and keeps no per-call state, so calls on
 *   different streams may run concurrently on different buffers. Device
 *   work is enqueued on the given HIP stream (NULL = the null stream) and
 *   is asynchronous: no call synchronises, and a device fault surfaces at
 *   the caller's next synchronisation. Errors found on the host are
 *   returned before anything is enqueued. No entry point throws.
 *
 * There is no dense fallback: inputs the kernels cannot take return an
 * error code and the caller decides what to do.
 */
#ifndef VSA_H
#define VSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. 0 is success; errors are negative. */
enum {
  VSA_OK = 0,
  VSA_ERR_INVALID_ARG = -1,  /* null pointer, a size <= 0, prefix_len < 0   */
  VSA_ERR_TOPK = -2,         /* topk < 1 or topk > num_blocks (the user
                                guide: top-k must be positive and may not
                                exceed the block count)                     */
  VSA_ERR_UNSUPPORTED = -3,  /* head_dim not 64 or 128, dtype unknown,  
                                cube volume > 1024, num_blocks > 4096       */
  VSA_ERR_ALIGN = -4,        /* pointer or stride not 16-byte aligned       */
  VSA_ERR_OVERFLOW = -5,     /* an element offset or a count would overflow
                                the kernels' index types                    */
  VSA_ERR_DEVICE = -6,       /* current device is not gfx950, or a HIP
                                query failed                                */
  VSA_ERR_LAUNCH = -7,       /* a kernel launch reported an error           */
  VSA_ERR_SCRATCH = -8       /* vsa_forward_noalloc: the problem needs more
                                scratch (plan.workspace_bytes) than its
                                fixed device array (32 MiB) holds           */
};

/* Element type of q, k, v and o. Softmax, row sums and the output
   accumulator are float32 for both; P is rounded to the input type before
   it multiplies V. */
enum { VSA_DTYPE_BF16 = 0, VSA_DTYPE_F16 = 1 };

/* What the caller asks for. All sizes in elements or tokens. */
typedef struct vsa_problem {
  int32_t batch;          /* B  >= 1                                         */
  int32_t heads;          /* Hh >= 1 (q, k and v have equal head counts)     */
  int32_t head_dim;       /* D: 64 or 128                                    */
  int32_t latent[3];      /* (T, H, W) grid, each >= 1                       */
  int32_t cube[3];        /* (ct, ch, cw) block shape, each >= 1            */
  int32_t topk;           /* cubes kept per query block, 1..num_blocks       */
  int32_t prefix_len;     /* P >= 0 tokens before the grid, always kept      */
  int32_t dtype;          /* VSA_DTYPE_BF16 or VSA_DTYPE_F16                 */
  int64_t stride_b, stride_h, stride_n;        /* q strides (elements), all
                                                  >= 1, or all 0: contiguous
                                                  [B][Hh][N][D]; k and v too
                                                  unless kv_stride_* set      */
  int64_t o_stride_b, o_stride_h, o_stride_n;  /* o strides (elements), or all
                                                  0: the same as q's          */
  /* k and v on a grid of their own (fastbsa package page, section "Use":
     latent_shape_k and chunk_3d_shape_k next to q's shapes). Each group
     all zero means "same as q". Query blocks then come from (latent, cube),
     key blocks from (latent_k, cube_k); prefix_len counts leading tokens of
     both sequences, each side cutting its prefix by its own cube volume. */
  int32_t latent_k[3];    /* (T, H, W) of k and v, each >= 1, or all 0      */
  int32_t cube_k[3];      /* key cube shape, each >= 1, or all 0            */
  int64_t kv_stride_b, kv_stride_h, kv_stride_n;  /* k, v strides, or all 0:
                             q's on q's grid, else contiguous [B][Hh][N_k][D] */
} vsa_problem;

/* Derived geometry; filled by vsa_plan, plain data, owned by the caller.
   p holds the problem with every defaulted group filled in (never zero). */
typedef struct vsa_plan_t {
  vsa_problem p;
  int32_t nblk[3];            /* query cubes per axis: ceil(T/ct), ceil(H/ch), ceil(W/cw) */
  int32_t num_blocks;         /* key cubes nT_k*nH_k*nW_k: the ids sel holds
                                 (equal to the query cube count when k and v
                                 share q's grid and cube)                   */
  int32_t num_prefix_blocks;  /* query prefix blocks ceil(P / V)             */
  int32_t num_q_blocks;       /* num_prefix_blocks + query cubes             */
  int32_t cube_volume;        /* V = ct*ch*cw                                */
  int64_t seq_len;            /* N = P + T*H*W tokens of q and o             */
  int64_t workspace_bytes;    /* bytes of float32 workspace vsa_select needs */
  int64_t kbar_offset;        /* byte offset of kbar inside the workspace    */
  int64_t sel_elems;          /* B*Hh*num_q_blocks*topk                      */
  float scale;                /* head_dim^-1/2                               */
  int32_t select_rows;        /* query blocks per score/top-k workgroup      */
  int32_t attend_variant;     /* attention kernel tiling chosen by the plan  */
  int32_t attend_tiles;       /* query row tiles per query block             */
  int32_t nblk_k[3];          /* key cubes per axis                          */
  int32_t num_prefix_blocks_k;/* key prefix blocks ceil(P / V_k), all kept   */
  int32_t cube_volume_k;      /* V_k                                         */
  int64_t seq_len_k;          /* N_k = P + T_k*H_k*W_k tokens of k and v     */
} vsa_plan_t;

/* Validate a problem and derive its geometry. Host only: no device work,
 * no allocation. Returns VSA_OK and fills *out, or an error code and leaves
 * *out unspecified. The Wan routing-log shape (31, 22, 40) with (4, 8, 8)
 * cubes gives num_blocks = 120 (user guide, "Wan top-k behavior"). */
int vsa_plan(const vsa_problem* problem, vsa_plan_t* out);

/* Top-k for a sparsity s in [0, 1), the fraction of key cubes dropped
 * (fastbsa package page, section "Use": sparsity=0.9375 keeps 1/16):
 * floor(num_blocks * (1 - s)), at least 1, so the kept fraction never
 * exceeds 1 - s; a product within 1e-9 (relative) of an integer counts as
 * that integer (decimal sparsities are not exact in binary). Returns it, or
 * VSA_ERR_INVALID_ARG for num_blocks < 1 or s outside [0, 1) (NaN
 * included). Host only. */
int vsa_topk_for_sparsity(int32_t num_blocks, double sparsity);

/* Block selection (pages: user guide opening definition; fastbsa "How it
 * works": the score matrix never leaves on-chip memory). Pools q over every
 * query block and k over every cube into the workspace, then scores every
 * query block against every cube and writes its topk cube ids, ascending,
 * to sel. q, k: device bf16/fp16 (plan dtype) per the plan's strides. workspace: device,
 * >= plan->workspace_bytes, 256-byte aligned. sel: device int32,
 * plan->sel_elems. stream: hipStream_t or NULL. Asynchronous. */
int vsa_select(const vsa_plan_t* plan, const void* q, const void* k,
               void* workspace, int32_t* sel, void* stream);

/* The two steps of vsa_select, for callers that time them apart or reuse
 * the pooled means. vsa_pool writes qbar and kbar into the workspace (same
 * arguments and rules as vsa_select); vsa_score_topk reads them from the
 * workspace and writes sel. vsa_select is vsa_pool then vsa_score_topk on
 * the same stream. Asynchronous. */
int vsa_pool(const vsa_plan_t* plan, const void* q, const void* k,
             void* workspace, void* stream);
int vsa_score_topk(const vsa_plan_t* plan, const void* workspace,
                   int32_t* sel, void* stream);

/* Block-sparse attention (pages: user guide opening definition; fastbsa
 * "How it works": raster-to-block index map evaluated inside the kernel).
 * For every query token, exact softmax attention over the tokens of all
 * prefix blocks and of the cubes listed in sel for its query block; o is
 * written in the same raster layout as q (o_stride_*). sel must hold valid
 * ascending ids as vsa_select writes them (other contents give undefined
 * output but stay in bounds: ids are clamped to 0..num_blocks-1). o must
 * not alias q, k or v. Asynchronous. */
int vsa_attend(const vsa_plan_t* plan, const void* q, const void* k,
               const void* v, const int32_t* sel, void* o, void* stream);

/* vsa_select followed by vsa_attend on the same stream. */
int vsa_forward(const vsa_plan_t* plan, const void* q, const void* k,
                const void* v, void* workspace, int32_t* sel, void* o,
                void* stream);

/* Grid sides for vsa_block_counts. */
enum { VSA_SIDE_Q = 0, VSA_SIDE_K = 1 };

/* Valid token count of every block of one side's grid, in block-id order:
 * the prefix blocks (V tokens each, the last one the remainder of the
 * prefix), then the cubes in raster order of the cube grid (a cube at the
 * far edge of an axis holds only the tokens inside the grid). side
 * VSA_SIDE_Q: q's grid (num_q_blocks entries); VSA_SIDE_K: the key grid
 * (num_prefix_blocks_k + num_blocks entries). Writes min(len, count)
 * entries to counts (host memory, caller-owned; may be NULL when len is 0)
 * and returns the count, or VSA_ERR_INVALID_ARG (null plan, unknown side,
 * len < 0) or vsa_plan's error for a plan that is not valid. Host only
 * (user guide, "Wan top-k behavior": 120 cubes for the (31, 22, 40) grid
 * in (4, 8, 8) blocks, the edge cubes partial). */
int vsa_block_counts(const vsa_plan_t* plan, int32_t side, int32_t* counts, int64_t len);

/* vsa_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation and kernels, with the pooled means kept
 * in a fixed array of 32 MiB of device memory
 * that the library holds on each device it runs on, from its first use
 * there until the process ends, instead of a caller workspace. The caller
 * still passes q, k, v, sel and o as for vsa_forward. Problems with
 * plan->workspace_bytes above 32 MiB (32 heads of 960 cubes of 64 tokens
 * need 31.5 MB; the Wan-shaped call 2.9 MB) return VSA_ERR_SCRATCH before any
 * device work. The call itself allocates nothing (no hipMalloc, hipFree or
 * allocating library routine). Every call on one device shares that
 * device's array: calls that overlap in time on one device (different
 * streams, or host threads) race and give undefined results; calls in one
 * stream order are safe. Asynchronous. */
int vsa_forward_noalloc(const vsa_plan_t* plan, const void* q, const void* k,
                        const void* v, int32_t* sel, void* o, void* stream);

/* Formats the routing fields of the user guide's Wan log line
 * ("seq_len=..., dit_seq_shape=(T, H, W), block_size=(ct, ch, cw),
 * num_blocks=..., topk=..., keep_ratio=..%") into buf (always
 * NUL-terminated when len > 0). Returns the length the full string needs,
 * excluding the NUL, or a negative error code. */
int vsa_describe(const vsa_plan_t* plan, char* buf, size_t len);

/* Static description of a status code; never NULL. */
const char* vsa_status_str(int status);

/* ---- Routing front end (user guide, sections "Wan top-k behavior" and
 * "Verify routing and fallback"). Host only, no device work. The library
 * itself never runs dense attention: a DENSE route tells the caller to run
 * its own dense attention, for the reason given. */
enum {
  VSA_ROUTE_VSA = 0,             /* top-k block selection ("route=VSA")        */
  VSA_ROUTE_VSA_ALL_BLOCKS = 1,  /* every block through the sparse kernels
                                    ("route=VSA_ALL_BLOCKS")                   */
  VSA_ROUTE_DENSE = 2            /* dense attention by the caller ("route=SDPA") */
};
enum {
  VSA_CHECKPOINT_NATIVE = 0,     /* topk == num_blocks goes dense: scoring every
                                    block gives no sparsity benefit            */
  VSA_CHECKPOINT_DMD = 1         /* topk == num_blocks stays on the sparse
                                    kernels (the checkpoint was trained with
                                    them)                                     */
};
enum {
  VSA_REASON_NONE = 0,
  VSA_REASON_TOPK_ABOVE_BLOCKS = 1,  /* topk > num_blocks for this shape      */
  VSA_REASON_ALL_BLOCKS_NATIVE = 2,  /* topk == num_blocks, native checkpoint */
  VSA_REASON_UNSUPPORTED = 3         /* vsa_plan refused the problem; status
                                        holds its code                        */
};

typedef struct vsa_route_t {
  int32_t route;            /* VSA_ROUTE_*                                   */
  int32_t reason;           /* VSA_REASON_*                                  */
  int32_t status;           /* vsa_plan's status for VSA_REASON_UNSUPPORTED  */
  int32_t checkpoint_mode;  /* as passed                                     */
  int32_t topk;             /* as asked (may exceed plan.num_blocks)         */
  int32_t has_plan;         /* 1: plan holds the problem's geometry (for a
                               top-k above the block count, planned with
                               topk = num_blocks); 0: no geometry            */
  vsa_plan_t plan;          /* ready for vsa_select / vsa_attend when route
                               is VSA or VSA_ALL_BLOCKS                      */
} vsa_route_t;

/* Decide the route of one problem. Returns VSA_OK and fills *out, or
 * VSA_ERR_INVALID_ARG (null pointer, unknown checkpoint mode) or
 * VSA_ERR_TOPK (topk < 1: a configuration error, not a fallback). */
int vsa_route(const vsa_problem* problem, int32_t checkpoint_mode, vsa_route_t* out);

/* The routing log line for a route ("FASTVIDEO_VSA routing: seq_len=...,
 * ..., keep_ratio=..%, checkpoint_mode=native, route=VSA", with
 * ", reason=..." on a dense route), the same fields and order as the user
 * guide's Wan log. Writes into buf like vsa_describe and returns the full
 * length, or a negative error code. */
int vsa_describe_route(const vsa_route_t* route, char* buf, size_t len);

#ifdef __cplusplus
}
#endif

#endif /* VSA_H */
