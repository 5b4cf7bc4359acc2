// Persistent whole-stack sweep for decode-sized M (one cooperative launch).
#pragma once

#include <vector>

#include "lb_internal.h"

struct lb_layer;

namespace lbi {

struct PersistPlan;

// Build the device program for a stack; LB_EUNSUPPORTED when the device or
// the shapes cannot run it (the caller then uses per-layer kernels).
lb_status persist_build(const std::vector<lb_layer *> &layers, const std::vector<int> &unit_begin,
                        const std::vector<int> &unit_size, float kappa, int device,
                        PersistPlan **out);
void persist_free(PersistPlan *p);
int64_t persist_max_rows();
lb_status persist_run(PersistPlan *p, const uint16_t *x0, uint16_t *y, uint16_t *const *traceY,
                      uint16_t *const *traceX, int64_t M, hipStream_t st);

}  // namespace lbi
