// plan.h -- host planner interface (internal to the library).
#pragma once

#include <cstdint>

#include "../../include/gemm.h"

namespace dgw {

// Fill *out for a call of `batch` (>= 1) products; returns a GEMM_* status and
// points *why at a message.
int make_plan(int64_t M, int64_t N, int64_t K, int64_t batch, uint32_t layout, uint32_t mode, int32_t splits,
              int32_t num_cus, gemm_plan_t *out, const char **why);

// Fill *out for a grouped call (only M and N of the groups are read): the plan
// of one problem with the same tile count, with the workspace of the groups'
// Split-K partials and their table (group_table_bytes(count) at its end).
int make_plan_grouped(const gemm_group_t *groups, int32_t count, int64_t K, uint32_t layout, uint32_t mode,
                      int32_t splits, int32_t num_cus, gemm_plan_t *out, const char **why);
int64_t group_table_bytes(int32_t count);

// The mode word with GEMM_TILE_AUTO replaced by the tile it picks for this call
// (any other mode word comes back unchanged).
uint32_t choose_tile(int64_t M, int64_t N, int64_t K, int64_t batch, uint32_t layout, uint32_t mode, int32_t splits,
                     int32_t num_cus);
uint32_t choose_tile_grouped(const gemm_group_t *groups, int32_t count, int64_t K, uint32_t layout, uint32_t mode,
                             int32_t splits, int32_t num_cus);

// First flattened iteration of Stream-K unit `unit` ("big" units first).
int64_t unit_begin(int64_t unit, int64_t q, int64_t big);

// Bytes of control words (status, flags, counters) at the head of the workspace.
int64_t control_bytes(const gemm_plan_t &p);

}  // namespace dgw
