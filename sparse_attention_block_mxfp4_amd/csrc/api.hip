// Status reporting and the configuration guard of the C ABI.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "common.h"

static thread_local char g_err[512] = "";

void mi_idx_clear_error() { g_err[0] = '\0'; }

int mi_idx_fail(int status, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return status;
}

int mi_idx_check_launch(const char *what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return mi_idx_fail(MI_IDX_EHIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return MI_IDX_OK;
}

extern "C" const char *mi_idx_version(void) { return "mi_idx 0.1 gfx950"; }

extern "C" const char *mi_idx_last_error(void) { return g_err; }

extern "C" const char *mi_idx_unsupported_reason(int topk_blocks, int init_blocks,
                                                 int local_blocks, int block_size,
                                                 int head_dim, const char *score_type,
                                                 int num_heads, int max_query_len) {
  if (topk_blocks != MI_IDX_TOPK || init_blocks != 0 || local_blocks != 1 ||
      block_size != MI_IDX_PAGE_TOKENS || head_dim != MI_IDX_HEAD_DIM ||
      score_type == nullptr || strcmp(score_type, "max") != 0)
    return "needs topk_blocks=16, init_blocks=0, local_blocks=1, block_size=128, "
           "index_head_dim=128 and score_type='max'";
  if (num_heads < 1 || num_heads > MI_IDX_MAX_HEADS)
    return "serves 1..8 index heads per call";
  if (max_query_len < 1 || max_query_len > MI_IDX_MAX_QUERY_LEN)
    return "scores at most 8 decode queries per request";
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return "needs a HIP device";
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    (void)hipGetLastError();
    return "needs a HIP device";
  }
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) return "needs gfx950";
  return nullptr;
}
