// Device top-k over a score array: the launcher the rerank entry points share with the
// standalone maxsim_topk entry (implemented in maxsim_topk.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace maxsim {

constexpr int kTopkMaxK = 1024;

// Workspace bytes of launch_topk for B scores and k results (256-byte multiple).
size_t topk_workspace_bytes(int32_t B, int32_t k);

// Enqueue the selection of the k best of scores[0, B) into top_scores / top_ids
// (0 < k <= kTopkMaxK; arguments already checked). Returns a MAXSIM_* status.
int launch_topk(const float *scores, int32_t B, int32_t k, float *top_scores, int32_t *top_ids, char *ws,
                hipStream_t stream);

}  // namespace maxsim
