// Host-side internals shared by api.cpp and plan.cpp.
#pragma once
#include <hip/hip_runtime.h>

#include "../../include/libjolt.h"
#include "dev_common.h"
#include "payload.h"
#include "planner.h"

#include <vector>

struct jolt_handle_s;

namespace jolt {

jolt_status fail(jolt_handle h, jolt_status s, const char *fmt, ...);
jolt_status hip_fail(jolt_handle h, hipError_t e, const char *where);
void clear_err(jolt_handle h);
// The dual's candidate grid and per-shape byte-ordered candidates depend only
// on the configuration and the item shapes; a handle keeps the last ones from
// one plan to the next.
struct DualTables {
    int rt_max = -1, rf_max = -1, step = -1, grid_nf = -1, dtype = -1, d = -1;
    uint32_t bits_mask = 0;
    std::vector<Cand> cand;
    std::vector<int> cell;          // each candidate's energy-grid cell (-1 for rank 0)
    struct Shape {
        int L, H, T;
        SortedCands sc;             // the candidates in byte order, with their bytes
    };
    std::vector<Shape> shapes;
};
DualTables &dual_tables(jolt_handle h);
// The handle's pinned host buffer of at least `bytes` (grown on demand) for a
// device-to-host copy that the caller synchronises before it returns.
hipError_t readback_buffer(jolt_handle h, size_t bytes, uint8_t **buf);
// The handle's small pinned host buffer (2 kMaxBatch floats) for the block
// Jacobi convergence norms, read once per sweep.
hipError_t sweep_buffer(jolt_handle h, float **buf);
// A second stream on the handle's device (default priority, created on first
// use and destroyed with the handle) and two events, for work forked off the
// caller's stream and joined back to it within one call.
hipError_t side_stream(jolt_handle h, hipStream_t *st, hipEvent_t *fork, hipEvent_t *join);
// Waits for the handle's side stream (if it exists): an error path's
// guarantee that nothing it launched still runs.
void drain_streams(jolt_handle h);
jolt_status check_item(jolt_handle h, const jolt_item &it);
jolt_status check_alloc(jolt_handle h, const jolt_item &it, const jolt_alloc &a);
jolt_status check_items_uniform(jolt_handle h, const jolt_item *items, int n);

// plan.cpp
jolt_status check_config(jolt_handle h, const jolt_config &cfg, const jolt_item *items, int n);
jolt_status store_params(jolt_handle h, const PlanLayout &pl, const jolt_item *items, int n, const jolt_alloc *alloc,
                         const void *plan_ws, void *const *payload_dev, hipStream_t st);

}  // namespace jolt
