// Persistent whole-stack sweep for decode-sized M: one launch of one
// workgroup per compute unit, all of which must be resident at once.
#pragma once

#include <string>
#include <vector>

#include "lb_internal.h"

namespace lbi {

struct PersistPlan;

// Build the device program for a stack; LB_EUNSUPPORTED when the device or
// the shapes cannot run it (the caller then uses per-layer kernels).
lb_status persist_build(const std::vector<lb_layer *> &layers, const std::vector<int> &unit_begin,
                        const std::vector<int> &unit_size, float kappa, int device,
                        PersistPlan **out);
void persist_free(PersistPlan *p);
int64_t persist_max_rows();
// Launch the sweep for M rows (M <= persist_max_rows()).  trace, when not
// null, receives every layer's output then every unit's input (M = 1).
lb_status persist_run(PersistPlan *p, const uint16_t *x0, uint16_t *y, uint16_t *trace, int64_t M,
                      hipStream_t st, std::string *msg);
// Diagnostics: per-phase device timestamps of every workgroup.
void persist_set_timeline(PersistPlan *p, uint64_t *buf);
// Failure test: later sweeps wait for a generation nobody writes, with a
// short bound, so every wait gives up and sets the error word.
void persist_set_fail_test(PersistPlan *p, bool on);
// Stress test: later sweeps delay each wave at the exchange's steps by a
// pseudo-random time of up to max_ticks ticks of 10 ns (0 = off).
void persist_set_delay(PersistPlan *p, unsigned seed, unsigned max_ticks);
int persist_grid(const PersistPlan *p);
int persist_phases(const PersistPlan *p);
int persist_stamps();  // timestamps per phase and workgroup
// Synchronise and report a device-side wait timeout of an earlier launch.
lb_status persist_check(PersistPlan *p, std::string *msg);

}  // namespace lbi
