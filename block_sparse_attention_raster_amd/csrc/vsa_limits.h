// Internal limits and tiling codes shared by the host plan and the launchers.
#ifndef VSA_LIMITS_H
#define VSA_LIMITS_H

#define VSA_MAX_CUBE_VOLUME 1024      /* tokens per block                      */
#define VSA_MAX_BLOCKS 4096           /* video cubes per (batch, head): four
                                         score rows of 4096 keys fill the
                                         selection LDS budget               */
#define VSA_SELECT_MAX_ROWS 16        /* query blocks per score/top-k group    */
#define VSA_SELECT_SCORE_LDS 65536    /* bytes of LDS for one group's scores   */
#define VSA_SELECT_MFMA_MAX_BLOCKS 2048 /* cubes scored on the matrix cores    */
#define VSA_NOALLOC_SCRATCH_BYTES (32u << 20) /* device scratch of the
                                         allocation-free entry point: the
                                         pooled means of plan.workspace_bytes
                                         (31.5 MB for 32 heads of 960 cubes) */

enum {
  VSA_ATTEND_ROWS64 = 1,   /* 64 query rows per workgroup (cubes <= 64 tokens) */
  VSA_ATTEND_ROWS256 = 2   /* 256 query slots per workgroup (8 waves)          */
};

#endif
